"""Oracle: attention over a paged KV cache, in float64 (test infrastructure only).

What is computed (the plain definition; paging is only an address translation):

* Paging [P3 §"Anatomy of the KV Cache: Memory Layout, Paging and Quantization Trade-offs";
  P1 §"PagedAttention: making the KV cache schedulable"; P5 §"PagedAttention: The Other Half
  of the Story"]: physical KV memory is a pool of fixed-size blocks laid out
  [num_blocks, block_size, num_heads, head_dim]; each sequence owns a block table listing block
  ids in logical order, so logical position j lives in block ``table[j // block_size]`` at row
  ``j % block_size``.  The pool here holds one such plane for K and one for V.
* Decode and verify rows [P1 §"The core idea"; P2 §"Speculative Decoding: Draft Fast, Verify
  Cheap"; P3 §"Speculative Decoding: Turning Verification Parallelism into Latency Wins"]: a
  sequence with context length L (counting this step's Q new tokens) brings Q query rows; row i
  sits at absolute position L - Q + i and sees keys 0 .. L - Q + i (causal within the draft or
  prefill chunk), so the Q rows equal Q sequential single-token decode steps.
* Grouped-query attention [P3 §"Prefill vs. Decode: Two Distinct Bottlenecks"]: query head h
  reads KV head h // (Hq / Hkv).
* Scores use the scale 1/sqrt(head_dim) unless a scale is given; weights are the softmax of the
  scores over the visible keys; the output is the weighted sum of V rows.

* Tree-masked verification [P4 §"4. Tree Attention & Medusa Heads"; P3 §"Draft Model
  Selection and Tree-Style Variants"]: the draft is a token tree verified in one pass under a
  tree attention mask.  Read here as: a sequence's Q new rows are the tree's nodes in an order
  where every node follows its ancestors; node i sees the committed prefix (keys
  0 .. L - Q - 1) and the nodes j whose bit j is set in its mask (its ancestors and itself).
  A chain (mask_i = bits 0..i) is the causal verify above.
* 8-bit KV [P3 §"Quantization and Precision Choices for KV"]: INT8 KV needs per-head or
  per-token scale factors and dequantisation inside the attention kernel, with asymmetric
  quantisation and separate scales for K and V.  Read here as affine uint8 codes with one
  (scale, zero point) pair per token, KV head and plane: value = scale * (code - zero_point).
  Attention over such a cache is the plain definition above applied to the dequantised values.
* FP8 KV [P3 §"Quantization and Precision Choices for KV" names FP8 beside INT8]: codes are
  8-bit floats in the E4M3 format (OCP FP8), with the same per-token and per-head scale pairs:
  value = scale * (e4m3(code) - zero_point), the zero point 0 for a symmetric cache.

Reading taken where the pages are silent: the scale, the head grouping (contiguous groups) and
"L counts the new tokens" are the plainest readings consistent with the pages; for 8-bit KV,
the finer of the two granularities the pages name (per token and head) and the affine form.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (bf16 is the upper half of an IEEE fp32)."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def physical_slots(table_row: np.ndarray, n_tokens: int, block_size: int) -> np.ndarray:
    """Flat pool slot (block * block_size + row) of logical positions 0 .. n_tokens-1."""
    j = np.arange(n_tokens)
    blocks = np.asarray(table_row)[j // block_size].astype(np.int64)
    if n_tokens and (blocks.min() < 0):
        raise ValueError("block table entry < 0 inside the context")
    return blocks * block_size + (j % block_size)


def gather_sequence_kv(pool_plane: np.ndarray, table_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """Contiguous [n_tokens, Hkv, D] view of one sequence's K (or V) read through its table.

    ``pool_plane`` is [num_blocks, block_size, Hkv, D] of any dtype; rows are returned as-is.
    """
    nb, bs = pool_plane.shape[0], pool_plane.shape[1]
    flat = pool_plane.reshape(nb * bs, *pool_plane.shape[2:])
    return flat[physical_slots(table_row, n_tokens, bs)]


def attend_row(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * keys @ q_row) @ values for one query row over its visible keys.

    keys, values: [n, D] float64 with n >= 1.  The maximum score is subtracted before the
    exponential (a shift that leaves the softmax unchanged).
    """
    z = scale * (keys @ q_row)
    w = np.exp(z - z.max())
    return (w @ values) / w.sum()


def visible_keys(L: int, Q: int, i: int, tree_mask=None) -> np.ndarray:
    """Key positions row i of a sequence may attend: the causal range 0 .. L-Q+i, or with a
    tree mask the prefix 0 .. L-Q-1 plus L-Q+j for every bit j set in tree_mask[i]."""
    if tree_mask is None:
        return np.arange(L - Q + i + 1)
    m = int(tree_mask[i])
    nodes = [j for j in range(Q) if (m >> j) & 1]
    return np.concatenate([np.arange(L - Q), L - Q + np.asarray(nodes, dtype=np.int64)]).astype(np.int64)


def attention_sequence(q_seq: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray,
                       scale: float | None = None, heads=None, rows=None, tree_mask=None) -> np.ndarray:
    """Attention for one sequence with contiguous KV.

    q_seq [Q, Hq, D]; k_seq, v_seq [L, Hkv, D] (float64); tree_mask optional [Q] integers
    (``visible_keys``).  Returns [Q, Hq, D] float64 (entries not requested through ``rows`` /
    ``heads`` are left as NaN).
    """
    Q, Hq, D = q_seq.shape
    L, Hkv, _ = k_seq.shape
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if not 1 <= Q <= L:
        raise ValueError("need 1 <= q_len <= ctx_len")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.full((Q, Hq, D), np.nan)
    for i in (range(Q) if rows is None else rows):
        if tree_mask is None:
            sel = slice(0, L - Q + i + 1)    # keys 0 .. L-Q+i
        else:
            sel = visible_keys(L, Q, i, tree_mask)
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            out[i, h] = attend_row(q_seq[i, h], k_seq[sel, g], v_seq[sel, g], scale)
    return out


def paged_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                    block_tables: np.ndarray, ctx_lens, q_lens, scale: float | None = None) -> np.ndarray:
    """Attention for a ragged batch through block tables.

    q [T, Hq, D] float64 with rows packed by sequence; k_pool, v_pool [NB, bs, Hkv, D] float64;
    block_tables [B, MB] int; ctx_lens, q_lens [B].  Returns [T, Hq, D] float64.
    """
    out = np.empty(q.shape, dtype=np.float64)
    row = 0
    for s in range(len(ctx_lens)):
        L, Q = int(ctx_lens[s]), int(q_lens[s])
        ks = gather_sequence_kv(k_pool, block_tables[s], L)
        vs = gather_sequence_kv(v_pool, block_tables[s], L)
        out[row:row + Q] = attention_sequence(q[row:row + Q], ks, vs, scale)
        row += Q
    return out


def dequantize_u8(codes: np.ndarray, scale: np.ndarray, zero_point: np.ndarray) -> np.ndarray:
    """Affine 8-bit dequantisation in float64: scale * (code - zero_point).

    codes [..., D] uint8; scale, zero_point [...] (one pair per token and KV head).
    """
    c = np.asarray(codes).astype(np.float64)
    return np.asarray(scale, np.float64)[..., None] * (c - np.asarray(zero_point, np.float64)[..., None])


def gather_sequence_kv_u8(codes: np.ndarray, kv_scales: np.ndarray, table_row: np.ndarray, n_tokens: int):
    """Dequantised contiguous K and V [n_tokens, Hkv, D] (float64) of one sequence.

    codes [2, NB, bs, Hkv, D] uint8; kv_scales [NB, Hkv, bs, 4] float32 holding
    (k_scale, k_zero, v_scale, v_zero) per block, KV head and row.
    """
    sc = np.transpose(np.asarray(kv_scales), (0, 2, 1, 3))     # [NB, bs, Hkv, 4]
    s = gather_sequence_kv(sc, table_row, n_tokens)             # [n, Hkv, 4]
    kc = gather_sequence_kv(codes[0], table_row, n_tokens)      # [n, Hkv, D]
    vc = gather_sequence_kv(codes[1], table_row, n_tokens)
    return dequantize_u8(kc, s[..., 0], s[..., 1]), dequantize_u8(vc, s[..., 2], s[..., 3])


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact float64 value of 8-bit floating-point codes in the E4M3 format (OCP FP8, "e4m3fn"):
    bit 7 is the sign, bits 6..3 the exponent with bias 7, bits 2..0 the mantissa.  Exponent 0
    holds subnormals m * 2^-9; exponent and mantissa all ones (0x7f, 0xff) is NaN; there are no
    infinities, so the largest magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((e == 0xF) & (c & 0x7 == 0x7), np.nan, sign * mag)


def dequantize_fp8(codes: np.ndarray, scale: np.ndarray, zero_point: np.ndarray) -> np.ndarray:
    """FP8 KV values in float64: scale * (e4m3 value of the code - zero_point), one (scale, zero)
    pair per token and KV head (zero points are 0 for a symmetric cache)."""
    x = e4m3_to_f64(codes)
    return np.asarray(scale, np.float64)[..., None] * (x - np.asarray(zero_point, np.float64)[..., None])


def gather_sequence_kv_fp8(codes: np.ndarray, kv_scales: np.ndarray, table_row: np.ndarray, n_tokens: int):
    """Dequantised contiguous K and V [n_tokens, Hkv, D] (float64) of one sequence from an FP8
    cache: codes [2, NB, bs, Hkv, D] uint8 holding E4M3 bits, kv_scales as for the 8-bit cache."""
    sc = np.transpose(np.asarray(kv_scales), (0, 2, 1, 3))     # [NB, bs, Hkv, 4]
    s = gather_sequence_kv(sc, table_row, n_tokens)
    kc = gather_sequence_kv(codes[0], table_row, n_tokens)
    vc = gather_sequence_kv(codes[1], table_row, n_tokens)
    return dequantize_fp8(kc, s[..., 0], s[..., 1]), dequantize_fp8(vc, s[..., 2], s[..., 3])


def _paged_rows(q_bits, ctx_lens, q_lens, scale, rows, sequence_kv, tree_mask=None) -> dict:
    """Attention of the requested (packed row, head) pairs; ``sequence_kv(s, L)`` returns the
    float64 [L, Hkv, D] keys and values of sequence s; ``tree_mask`` [T] per packed row."""
    T, Hq, D = q_bits.shape
    starts = np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))])
    wanted = None
    if rows is not None:
        wanted = {}
        for t, h in rows:
            s = int(np.searchsorted(starts, t, side="right") - 1)
            wanted.setdefault(s, []).append((int(t), int(h)))
    result = {}
    for s in range(len(ctx_lens)):
        if wanted is not None and s not in wanted:
            continue
        L, Q, r0 = int(ctx_lens[s]), int(q_lens[s]), int(starts[s])
        ks, vs = sequence_kv(s, L)
        qs = bf16_bits_to_f64(q_bits[r0:r0 + Q])
        tm = None if tree_mask is None else np.asarray(tree_mask)[r0:r0 + Q]
        if wanted is None:
            o = attention_sequence(qs, ks, vs, scale, tree_mask=tm)
            for i in range(Q):
                for h in range(Hq):
                    result[(r0 + i, h)] = o[i, h]
        else:
            for t, h in wanted[s]:
                o = attention_sequence(qs, ks, vs, scale, heads=[h], rows=[t - r0], tree_mask=tm)
                result[(t, h)] = o[t - r0, h]
    return result


def paged_attention_bf16(q_bits: np.ndarray, pool_bits: np.ndarray, block_tables: np.ndarray,
                         ctx_lens, q_lens, scale: float | None = None, rows=None, tree_mask=None) -> dict:
    """Same as ``paged_attention`` from bf16 bit patterns, converting only what is read.

    q_bits [T, Hq, D] uint16; pool_bits [2, NB, bs, Hkv, D] uint16.  ``rows`` optionally
    restricts the work to a list of (packed row t, head h) pairs; the result maps each computed
    (t, h) to its [D] float64 output.
    """
    def sequence_kv(s, L):
        return (bf16_bits_to_f64(gather_sequence_kv(pool_bits[0], block_tables[s], L)),
                bf16_bits_to_f64(gather_sequence_kv(pool_bits[1], block_tables[s], L)))
    return _paged_rows(q_bits, ctx_lens, q_lens, scale, rows, sequence_kv, tree_mask)


def paged_attention_u8(q_bits: np.ndarray, codes: np.ndarray, kv_scales: np.ndarray,
                       block_tables: np.ndarray, ctx_lens, q_lens, scale: float | None = None,
                       rows=None, tree_mask=None) -> dict:
    """``paged_attention_bf16`` over an 8-bit KV cache: codes [2, NB, bs, Hkv, D] uint8 and
    kv_scales [NB, Hkv, bs, 4] float32, dequantised (``dequantize_u8``) as they are read."""
    def sequence_kv(s, L):
        return gather_sequence_kv_u8(codes, kv_scales, block_tables[s], L)
    return _paged_rows(q_bits, ctx_lens, q_lens, scale, rows, sequence_kv, tree_mask)


def paged_attention_fp8(q_bits: np.ndarray, codes: np.ndarray, kv_scales: np.ndarray,
                        block_tables: np.ndarray, ctx_lens, q_lens, scale: float | None = None,
                        rows=None, tree_mask=None) -> dict:
    """``paged_attention_bf16`` over an FP8 (E4M3) KV cache: codes [2, NB, bs, Hkv, D] uint8 and
    kv_scales [NB, Hkv, bs, 4] float32, dequantised (``dequantize_fp8``) as they are read."""
    def sequence_kv(s, L):
        return gather_sequence_kv_fp8(codes, kv_scales, block_tables[s], L)
    return _paged_rows(q_bits, ctx_lens, q_lens, scale, rows, sequence_kv, tree_mask)
