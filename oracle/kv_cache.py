"""Oracle: writing a step's K/V into the paged cache and committing after verification
(test infrastructure only).

What is computed:

* Append [P3 §"Anatomy of the KV Cache: Memory Layout, Paging and Quantization Trade-offs"]:
  the Q new tokens of a sequence with context length L (L counting them) sit at positions
  L - Q .. L - 1; position j is row j % block_size of block table[j // block_size].  Their K and
  V rows ([Q, Hkv, D] each) are written there.
* 8-bit append [P3 §"Quantization and Precision Choices for KV"]: each (token, KV head) row of
  K and of V is quantised on its own (per-token scales, separate for K and V, asymmetric).
  Reading taken: the usual affine uint8 min/max rule, in float32 --
      lo = min(0, min x), hi = max(0, max x), scale = max((hi - lo) / 255, eps_fp32),
      zero = clip(round((0 - lo) / scale), 0, 255), code = clip(round(x * (1/scale)) + zero, 0, 255)
  with round-half-even; value = scale * (code - zero).  (0 is exactly representable.)  The zero
  point is an integer, stored as float +0 .. 255 (0 - lo, not -lo, so that lo = 0 gives +0).
* Commit [P3 §"Speculative Decoding: Turning Verification Parallelism into Latency Wins":
  rollback of the KV of rejected tokens; P2 §"Speculative Decoding: Draft Fast, Verify Cheap"]:
  after verifying Q = k + 1 rows (the last committed token and k drafts) with n accepted, the
  rejected drafts' K/V are dropped: the context length becomes L - Q + 1 + n.  For a draft tree
  the accepted nodes a_1 < ... < a_n (node 0 being the root at position L - Q) are first moved
  to positions L - Q + 1 .. L - Q + n, so the kept tokens are contiguous; a chain needs no move.
"""

from __future__ import annotations

import numpy as np

from .attention import physical_slots

FP32_EPS = np.float32(np.finfo(np.float32).eps)


def quantize_rows_u8(x: np.ndarray):
    """Affine uint8 quantisation of every row of x [..., D] (float32 arithmetic throughout).

    Returns (codes uint8 [..., D], scale float32 [...], zero float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    lo = np.minimum(x.min(axis=-1), np.float32(0))
    hi = np.maximum(x.max(axis=-1), np.float32(0))
    scale = np.maximum((hi - lo) / np.float32(255), FP32_EPS).astype(np.float32)
    zero = np.clip(np.rint((np.float32(0) - lo) / scale), 0, 255).astype(np.float32)   # +0, never -0
    inv = (np.float32(1) / scale).astype(np.float32)
    codes = np.clip(np.rint(x * inv[..., None]) + zero[..., None], 0, 255).astype(np.uint8)
    return codes, scale, zero


def _new_slots(table_row, L: int, Q: int, bs: int) -> np.ndarray:
    """Flat pool slots of positions L-Q .. L-1."""
    return physical_slots(table_row, L, bs)[L - Q:]


def kv_append(pool: np.ndarray, block_tables, ctx_lens, q_lens, k_new: np.ndarray, v_new: np.ndarray) -> np.ndarray:
    """Copy of pool [2, NB, bs, Hkv, D] (any dtype) with each sequence's new K/V rows written.

    k_new, v_new [T, Hkv, D] packed by sequence like the query rows.
    """
    out = np.array(pool, copy=True)
    NB, bs = out.shape[1], out.shape[2]
    flat = out.reshape(2, NB * bs, *out.shape[3:])
    row = 0
    for s in range(len(ctx_lens)):
        L, Q = int(ctx_lens[s]), int(q_lens[s])
        slots = _new_slots(block_tables[s], L, Q, bs)
        flat[0, slots] = k_new[row:row + Q]
        flat[1, slots] = v_new[row:row + Q]
        row += Q
    return out


def kv_append_u8(codes: np.ndarray, kv_scales: np.ndarray, block_tables, ctx_lens, q_lens,
                 k_new: np.ndarray, v_new: np.ndarray):
    """8-bit append: quantise every new (token, head) row of K and V and write codes and
    (k_scale, k_zero, v_scale, v_zero) (kv_scales [NB, Hkv, bs, 4]).  Returns copies."""
    codes = np.array(codes, copy=True)
    scales = np.array(kv_scales, copy=True)
    NB, bs = codes.shape[1], codes.shape[2]
    flat = codes.reshape(2, NB * bs, *codes.shape[3:])
    row = 0
    for s in range(len(ctx_lens)):
        L, Q = int(ctx_lens[s]), int(q_lens[s])
        slots = _new_slots(block_tables[s], L, Q, bs)
        for plane, x in ((0, k_new[row:row + Q]), (1, v_new[row:row + Q])):
            c, sc, z = quantize_rows_u8(x)                 # [Q, Hkv, D], [Q, Hkv]
            flat[plane, slots] = c
            blk, r = slots // bs, slots % bs
            for h in range(codes.shape[3]):
                scales[blk, h, r, 2 * plane] = sc[:, h]
                scales[blk, h, r, 2 * plane + 1] = z[:, h]
        row += Q
    return codes, scales


def committed_lengths(ctx_lens, q_lens, n_accepted) -> np.ndarray:
    """L - Q + 1 + n: the last committed token and the n accepted drafts stay cached."""
    return (np.asarray(ctx_lens, np.int64) - np.asarray(q_lens, np.int64) + 1
            + np.asarray(n_accepted, np.int64))


def kv_commit_tree(pool: np.ndarray, block_tables, ctx_lens, q_lens, path, n_accepted,
                   kv_scales: np.ndarray | None = None):
    """Move each sequence's accepted tree nodes to contiguous positions (path[s][:n] are node
    indices, node a at position L - Q + a) and return (pool, scales, new lengths).  For an
    8-bit cache the nodes' scales move with their codes."""
    pool = np.array(pool, copy=True)
    scales = None if kv_scales is None else np.array(kv_scales, copy=True)
    NB, bs = pool.shape[1], pool.shape[2]
    flat = pool.reshape(2, NB * bs, *pool.shape[3:])
    for s in range(len(ctx_lens)):
        L, Q, n = int(ctx_lens[s]), int(q_lens[s]), int(n_accepted[s])
        slots = physical_slots(block_tables[s], L, bs)
        src = slots[L - Q + np.asarray(path[s][:n], dtype=np.int64)]
        dst = slots[L - Q + 1 + np.arange(n)]
        rows = flat[:, src].copy()                     # read every source before writing
        flat[:, dst] = rows
        if scales is not None:
            srows = scales[src // bs, :, src % bs].copy()    # [n, Hkv, 4]
            scales[dst // bs, :, dst % bs] = srows
    return pool, scales, committed_lengths(ctx_lens, q_lens, n_accepted)
