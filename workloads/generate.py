"""Seeded input generators (no attention or sampling arithmetic lives here).

Every draw comes from ``numpy.random.Generator(PCG64(seed))`` in a fixed, documented order,
so a (config, seed) pair names one input exactly on any machine.

Attention inputs, in draw order:
  1. context lengths L_s and query lengths Q_s (per-config distribution),
  2. query values q ~ N(0, 1), fp32 rounded to bf16 (round-to-nearest-even),
  3. pool values K, V ~ N(0, 1) for every pool slot, rounded to bf16,
  4. a random permutation of pool blocks; sequence s takes the next ceil(L_s / bs) of them
     as its block table, in logical order.
Pool slots that no sequence owns, and the rows of a sequence's last block past L_s, are then
overwritten with a poison value (NaN by default) so that any read past ``ctx_len`` shows up.
Unused block-table entries are -1.

8-bit KV inputs (``kv_format="u8"``) replace step 3 by
  3a. codes for every pool slot, uint8 = clip(round(N(128, 40)), 0, 255),
  3b. per (block, KV head, token) the four fp32 numbers (k_scale, k_zero, v_scale, v_zero):
      scales uniform in [0.01, 0.03], zero points integers uniform in [112, 143].
They are drawn directly in that shape (no quantiser runs here); the scales of unowned slots and
of rows past L_s are poisoned instead of the codes.

FP8 KV inputs (``kv_format="fp8"``) replace step 3 by
  3a. codes for every pool slot: N(0, 1) values (fp32) rounded to the nearest E4M3 value (OCP
      FP8, ties to even, by torch's float8_e4m3fn conversion), stored as their uint8 bits,
  3b. per (block, KV head, token) (k_scale, 0, v_scale, 0): scales uniform in [0.5, 1.5] and
      zero points 0 (a symmetric cache).

New K/V rows of a step (``new_kv_rows``), in draw order: per (row, KV head) a spread
sigma ~ U[0.05, 4] and an offset mu ~ N(0, 0.5) for K, then the same for V; then K and V values
sigma * N(0, 1) + mu, rounded to bf16.  The varying ranges and signs exercise the 8-bit
quantiser's per-row scales and zero points.

Speculative-verification inputs, in draw order:
  1. logits (target rows [B, k+1, V], draft rows [B, k, V]) per the config,
  2. draft tokens x_i ~ q_i (one categorical draw per draft position),
  3. uniforms u in the open interval (0, 1), k+1 per sequence, exactly representable in fp32.
Probability rows are softmax(logits) evaluated in float64 and stored as float32; this is the
input recipe (the verifier consumes probabilities), not part of the verifier.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

CONFIG_NAMES = ("tiny", "llama3_8b_decode", "spec_verify_step", "llama70b_share", "mixed_step",
                "tree_verify_step")
DEFAULT_SEEDS = {name: 1001 + i for i, name in enumerate(CONFIG_NAMES)}

_CHUNK = 1 << 24  # values drawn per numpy call when filling large pools


@dataclass
class AttnInputs:
    """One ragged batch for a paged attention step (CPU tensors; move with ``.to(device)``).

    q            bf16  [T, Hq, D]     rows packed by sequence, in sequence order
    kv_pool      bf16  [2, NB, bs, Hkv, D]   plane 0 = K, plane 1 = V
                 (uint8 codes of the same shape when kv_scales is set)
    kv_scales    None, or fp32 [NB, Hkv, bs, 4] = (k_scale, k_zero, v_scale, v_zero) per token
    tree_mask    None, or int64 [T] (the bits of a uint64): bit j of a sequence's row i set when
                 row i may attend the sequence's new row j (tree verification)
    block_tables int32 [B, MB]        logical block -> physical block, -1 padded
    ctx_lens     int32 [B]            L_s, counting this step's Q_s new tokens
    q_lens       int32 [B]            Q_s (1 = decode, k+1 = verify, chunk = prefill)
    """

    name: str
    seed: int
    q: torch.Tensor
    kv_pool: torch.Tensor
    block_tables: torch.Tensor
    ctx_lens: torch.Tensor
    q_lens: torch.Tensor
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_scales: torch.Tensor | None = None
    tree_mask: torch.Tensor | None = None
    fp8: bool = False               # kv_pool holds E4M3 codes (kv_scales set) rather than uint8 codes

    @property
    def kv_format(self) -> str:
        return "bf16" if self.kv_scales is None else ("fp8" if self.fp8 else "u8")

    @property
    def num_seqs(self) -> int:
        return int(self.ctx_lens.numel())

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.kv_pool.shape[1])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


@dataclass
class VerifyInputs:
    """One batch for speculative verification (CPU tensors).

    p          fp32  [B, k+1, V]   target probabilities for the k drafts plus the bonus row
    q          fp32  [B, k, V]     draft probabilities
    draft_ids  int32 [B, k]
    uniforms   fp32  [B, k+1]      u[:, :k] for the accept tests, u[:, k] for the final draw
    """

    name: str
    seed: int
    p: torch.Tensor
    q: torch.Tensor
    draft_ids: torch.Tensor
    uniforms: torch.Tensor

    @property
    def num_seqs(self) -> int:
        return int(self.p.shape[0])

    @property
    def k(self) -> int:
        return int(self.q.shape[1])

    @property
    def vocab(self) -> int:
        return int(self.p.shape[2])


# ----------------------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------------------

def _normal_bf16(rng: np.random.Generator, shape) -> torch.Tensor:
    """N(0,1) fp32 draws rounded to bf16, drawn in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.bfloat16)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        x = rng.standard_normal(stop - start, dtype=np.float32)
        out[start:stop] = torch.from_numpy(x).to(torch.bfloat16)
    return out.view(*shape)


def _codes_u8(rng: np.random.Generator, shape) -> torch.Tensor:
    """uint8 codes clip(round(N(128, 40)), 0, 255), drawn in chunks."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.uint8)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        x = np.clip(np.rint(128.0 + 40.0 * rng.standard_normal(stop - start, dtype=np.float32)), 0, 255)
        out[start:stop] = torch.from_numpy(x.astype(np.uint8))
    return out.view(*shape)


def _scales_u8(rng: np.random.Generator, shape) -> torch.Tensor:
    """[..., 4] fp32 (k_scale, k_zero, v_scale, v_zero): scales U[0.01, 0.03], zeros U{112..143}."""
    n = int(np.prod(shape))
    sc = rng.uniform(0.01, 0.03, size=(n, 2)).astype(np.float32)
    zp = rng.integers(112, 143, size=(n, 2), endpoint=True).astype(np.float32)
    out = np.stack([sc[:, 0], zp[:, 0], sc[:, 1], zp[:, 1]], axis=1)
    return torch.from_numpy(out).view(*shape, 4)


def _codes_fp8(rng: np.random.Generator, shape) -> torch.Tensor:
    """uint8 bits of N(0, 1) values rounded to E4M3 (torch float8_e4m3fn), drawn in chunks."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.uint8)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        x = torch.from_numpy(rng.standard_normal(stop - start, dtype=np.float32))
        out[start:stop] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return out.view(*shape)


def _scales_fp8(rng: np.random.Generator, shape) -> torch.Tensor:
    """[..., 4] fp32 (k_scale, 0, v_scale, 0): scales U[0.5, 1.5], zero points 0."""
    n = int(np.prod(shape))
    sc = rng.uniform(0.5, 1.5, size=(n, 2)).astype(np.float32)
    z = np.zeros(n, np.float32)
    out = np.stack([sc[:, 0], z, sc[:, 1], z], axis=1)
    return torch.from_numpy(out).view(*shape, 4)


def open_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms in the open interval (0, 1): (j + 1/2) / 2^24, exactly representable in fp32."""
    j = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return ((j.astype(np.float64) + 0.5) / float(1 << 24)).astype(np.float32)


def random_tree_parents(rng: np.random.Generator, n: int) -> np.ndarray:
    """A random recursive tree of n nodes in topological order: node 0 is the root (parent -1),
    node i > 0 hangs under a parent drawn uniformly from 0 .. i-1."""
    par = np.full(n, -1, dtype=np.int64)
    for i in range(1, n):
        par[i] = rng.integers(0, i)
    return par


def tree_masks(parents) -> np.ndarray:
    """Ancestor masks of a tree in topological order: bit j of entry i is set when node j is
    node i or one of its ancestors.  Returned as int64 holding the uint64 bit pattern."""
    par = np.asarray(parents, dtype=np.int64)
    n = par.size
    assert n <= 64 and all(par[i] < i for i in range(n))
    masks = [0] * n
    for i in range(n):
        masks[i] = (1 << i) | (masks[par[i]] if par[i] >= 0 else 0)
    return np.array(masks, dtype=np.uint64).view(np.int64)


def _lognormal_lengths(rng, n, median, sigma, lo, hi):
    x = np.exp(math.log(median) + sigma * rng.standard_normal(n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def _pareto_lengths(rng, n, alpha, lmin, cap):
    u = rng.random(n)
    u = np.where(u <= 0.0, np.nextafter(0.0, 1.0), u)
    return np.minimum(np.floor(lmin * u ** (-1.0 / alpha)), cap).astype(np.int64)


# ----------------------------------------------------------------------------------------
# attention inputs
# ----------------------------------------------------------------------------------------

def make_attention_inputs(
    seed: int,
    *,
    ctx_lens,
    q_lens,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    max_ctx: int | None = None,
    pool_blocks: int | None = None,
    pool_factor: float = 1.2,
    poison: float = float("nan"),
    rng: np.random.Generator | None = None,
    name: str = "custom",
    kv_format: str = "bf16",
) -> AttnInputs:
    """Build one paged batch from given lengths (steps 2-4 of the draw order above).

    ``max_ctx`` fixes the block-table width (ceil(max_ctx / bs)); by default the realised
    maximum.  ``pool_blocks`` fixes the pool size; by default ceil(pool_factor * live blocks).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    L = np.asarray(ctx_lens, dtype=np.int64)
    Q = np.asarray(q_lens, dtype=np.int64)
    assert L.shape == Q.shape and L.ndim == 1
    assert np.all(Q >= 1) and np.all(L >= Q), "need 1 <= q_len <= ctx_len"
    B = L.size
    bs = int(block_size)
    nblk = (L + bs - 1) // bs
    live = int(nblk.sum())
    if max_ctx is None:
        max_ctx = int(L.max()) if B else bs
    MB = max(1, (int(max_ctx) + bs - 1) // bs)
    assert np.all(nblk <= MB)
    if pool_blocks is None:
        pool_blocks = max(live, int(math.ceil(pool_factor * live)))
    NB = int(pool_blocks)
    assert NB >= live
    T = int(Q.sum())

    q = _normal_bf16(rng, (T, num_q_heads, head_dim))
    scales = None
    if kv_format == "bf16":
        pool = _normal_bf16(rng, (2, NB, bs, num_kv_heads, head_dim))
    elif kv_format == "u8":
        pool = _codes_u8(rng, (2, NB, bs, num_kv_heads, head_dim))
        scales = _scales_u8(rng, (NB, num_kv_heads, bs))
    elif kv_format == "fp8":
        pool = _codes_fp8(rng, (2, NB, bs, num_kv_heads, head_dim))
        scales = _scales_fp8(rng, (NB, num_kv_heads, bs))
    else:
        raise ValueError(f"kv_format {kv_format!r}")
    perm = rng.permutation(NB)

    tables = np.full((B, MB), -1, dtype=np.int32)
    owned = np.zeros(NB, dtype=bool)
    cursor = 0
    for s in range(B):
        ids = perm[cursor:cursor + nblk[s]]
        cursor += int(nblk[s])
        tables[s, : nblk[s]] = ids
        owned[ids] = True
        tail = int(L[s] % bs)
        if tail:
            if scales is None:
                pool[:, int(ids[-1]), tail:] = poison
            else:
                scales[int(ids[-1]), :, tail:] = poison
    unused = np.nonzero(~owned)[0]
    if unused.size:
        if scales is None:
            pool[:, torch.from_numpy(unused)] = poison
        else:
            scales[torch.from_numpy(unused)] = poison

    return AttnInputs(
        name=name,
        seed=seed,
        q=q,
        kv_pool=pool,
        block_tables=torch.from_numpy(tables),
        ctx_lens=torch.from_numpy(L.astype(np.int32)),
        q_lens=torch.from_numpy(Q.astype(np.int32)),
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=bs,
        kv_scales=scales,
        fp8=kv_format == "fp8",
    )


_ATTN_SHAPES = {
    # name: (num_q_heads, num_kv_heads, head_dim, block_size, max_ctx)
    "tiny": (8, 2, 64, 16, 256),
    "llama3_8b_decode": (32, 8, 128, 16, 8192),
    "spec_verify_step": (32, 8, 128, 16, 4096),
    "llama70b_share": (64, 8, 128, 16, 32768),
    "mixed_step": (32, 8, 128, 32, 4096),
    "tree_verify_step": (32, 8, 128, 16, 4096),
}


def _config_lengths(name: str, rng: np.random.Generator):
    """Step 1 of the draw order: (ctx_lens, q_lens) of a named workload."""
    if name == "tiny":
        return np.array([17, 64, 100, 255]), np.ones(4, np.int64)
    if name == "llama3_8b_decode":
        return _lognormal_lengths(rng, 64, 1024, 1.0, 16, 8192), np.ones(64, np.int64)
    if name == "spec_verify_step":
        return rng.integers(512, 4096, size=16, endpoint=True), np.full(16, 5, np.int64)
    if name == "llama70b_share":
        return _pareto_lengths(rng, 256, 1.5, 128, 32768), np.ones(256, np.int64)
    if name == "mixed_step":
        Ld = _lognormal_lengths(rng, 128, 1024, 1.0, 16, 4096)
        Lv = _lognormal_lengths(rng, 32, 1024, 1.0, 16, 4096)
        Lp = rng.integers(256, 4096, size=4, endpoint=True)
        L = np.concatenate([Ld, Lv, Lp])
        Q = np.concatenate([np.ones(128, np.int64), np.full(32, 5, np.int64), np.full(4, 256, np.int64)])
        order = rng.permutation(L.size)
        return L[order], Q[order]
    if name == "tree_verify_step":
        return rng.integers(512, 4096, size=16, endpoint=True), np.full(16, 16, np.int64)
    raise KeyError(name)


def config_lengths(name: str, seed: int | None = None):
    """(ctx_lens, q_lens, (Hq, Hkv, D, bs, max_ctx)) of a named workload, without its tensors."""
    if seed is None:
        seed = DEFAULT_SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    L, Q = _config_lengths(name, rng)
    return L, Q, _ATTN_SHAPES[name]


def attention_config(name: str, seed: int | None = None, poison: float = float("nan"),
                     kv_format: str = "bf16") -> AttnInputs:
    """The five named attention workloads (lengths drawn first, then make_attention_inputs).

    tiny              4 decode seqs, L = {17, 64, 100, 255}, 8 q / 2 kv heads, D 64, bs 16
    llama3_8b_decode  64 decode seqs, L lognormal(median 1024, sigma 1) clipped [16, 8192],
                      32 q / 8 kv heads, D 128, bs 16, pool 1.2x live blocks
    spec_verify_step  16 verify seqs (q_len 5), L uniform in [512, 4096], 32/8 heads, D 128
    tree_verify_step  16 seqs verifying 16-node token trees (random recursive trees, drawn after
                      the pool), L uniform in [512, 4096], 32/8 heads, D 128
    llama70b_share    256 decode seqs, L Pareto(alpha 1.5, min 128) capped at 32768,
                      64 q / 8 kv heads, D 128, bs 16
    mixed_step        128 decode + 32 verify (q_len 5) + 4 prefill chunks (q_len 256);
                      decode/verify L lognormal(1024, 1) clipped [16, 4096], prefill L uniform
                      in [256, 4096]; 32/8 heads, D 128, bs 32; pool 95% full; order shuffled
    All other pools hold ceil(1.2 x live blocks).  ``kv_format="u8"`` gives the same lengths
    and shapes with 8-bit codes and per-token scales, ``kv_format="fp8"`` with E4M3 codes.
    """
    if seed is None:
        seed = DEFAULT_SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    L, Q = _config_lengths(name, rng)
    Hq, Hkv, D, bs, max_ctx = _ATTN_SHAPES[name]
    pool_blocks = None
    if name == "mixed_step":
        live = int(((L + bs - 1) // bs).sum())
        pool_blocks = int(math.ceil(live / 0.95))
    inp = make_attention_inputs(seed, ctx_lens=L, q_lens=Q, num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim=D, block_size=bs, max_ctx=max_ctx,
                                pool_blocks=pool_blocks, poison=poison, rng=rng, name=name,
                                kv_format=kv_format)
    if name == "tree_verify_step":
        inp.tree_mask = torch.from_numpy(np.concatenate([tree_masks(random_tree_parents(rng, int(q)))
                                                         for q in Q]))
    return inp


def new_kv_rows(seed: int, total_q: int, num_kv_heads: int, head_dim: int):
    """(k_new, v_new) bf16 [total_q, Hkv, D]: the K/V rows a step appends to the cache."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (total_q, num_kv_heads)
    sig = rng.uniform(0.05, 4.0, size=(2, *shape)).astype(np.float32)
    mu = (0.5 * rng.standard_normal((2, *shape))).astype(np.float32)
    out = []
    for plane in range(2):
        z = rng.standard_normal((*shape, head_dim), dtype=np.float32)
        x = z * sig[plane][..., None] + mu[plane][..., None]
        out.append(torch.from_numpy(x).to(torch.bfloat16))
    return out[0], out[1]


# ----------------------------------------------------------------------------------------
# speculative-verification inputs
# ----------------------------------------------------------------------------------------

def _softmax_rows_f64(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def make_verify_inputs(seed: int, *, p_logits: np.ndarray, q_logits: np.ndarray,
                       rng: np.random.Generator | None = None, name: str = "custom") -> VerifyInputs:
    """Probabilities from logits, drafts x_i ~ q_i, and open-interval uniforms."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    B, k1, V = p_logits.shape
    k = k1 - 1
    assert q_logits.shape == (B, k, V)
    p32 = _softmax_rows_f64(p_logits.astype(np.float64)).astype(np.float32)
    q32 = _softmax_rows_f64(q_logits.astype(np.float64)).astype(np.float32)
    return make_verify_from_probs(seed, p32, q32, rng=rng, name=name)


def make_verify_from_probs(seed: int, p32: np.ndarray, q32: np.ndarray,
                           rng: np.random.Generator | None = None, name: str = "custom") -> VerifyInputs:
    """Drafts x_i ~ q_i and uniforms for given fp32 probability rows."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    B, k1, V = p32.shape
    k = k1 - 1
    drafts = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):
            w = q32[b, i].astype(np.float64)
            drafts[b, i] = rng.choice(V, p=w / w.sum())
    u = open_uniforms(rng, (B, k + 1))
    return VerifyInputs(name=name, seed=seed, p=torch.from_numpy(np.ascontiguousarray(p32)),
                        q=torch.from_numpy(np.ascontiguousarray(q32)),
                        draft_ids=torch.from_numpy(drafts), uniforms=torch.from_numpy(u))


def verify_config(name: str, seed: int | None = None, batch: int | None = None) -> VerifyInputs:
    """Named verification workloads.

    tiny              B 4, k 4, V 1000; target and draft logits independent N(0, 2)
    spec_verify_step  B 16, k 4, V 128256; target logits N(0, 3); draft logits = target logits
                      of the first k positions + N(0, 0.7) noise
    ``batch`` overrides B (same recipe) for batch sweeps.
    """
    if seed is None:
        seed = DEFAULT_SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny":
        B, k, V = batch or 4, 4, 1000
        pl = 2.0 * rng.standard_normal((B, k + 1, V))
        ql = 2.0 * rng.standard_normal((B, k, V))
    elif name == "spec_verify_step":
        B, k, V = batch or 16, 4, 128256
        pl = 3.0 * rng.standard_normal((B, k + 1, V))
        ql = pl[:, :k] + 0.7 * rng.standard_normal((B, k, V))
    else:
        raise KeyError(name)
    return make_verify_inputs(seed, p_logits=pl, q_logits=ql, rng=rng, name=name)


# ----------------------------------------------------------------------------------------
# verification from logits
# ----------------------------------------------------------------------------------------

@dataclass
class LogitsVerifyInputs:
    """One batch for verification from logits (CPU tensors).

    zp         fp32  [B, k+1, V]   target logits for the k drafts plus the bonus row
    zq         fp32  [B, k, V]     draft logits
    temps      fp32  [B]           sampling temperature per sequence (0 = greedy)
    draft_ids  int32 [B, k]        x_i ~ softmax(zq_i / T) (the first argmax when T = 0)
    uniforms   fp32  [B, k+1]
    """

    name: str
    seed: int
    zp: torch.Tensor
    zq: torch.Tensor
    temps: torch.Tensor
    draft_ids: torch.Tensor
    uniforms: torch.Tensor

    @property
    def num_seqs(self) -> int:
        return int(self.zp.shape[0])

    @property
    def k(self) -> int:
        return int(self.zq.shape[1])

    @property
    def vocab(self) -> int:
        return int(self.zp.shape[2])


def make_logits_verify_inputs(seed: int, zp: np.ndarray, zq: np.ndarray, temps,
                              rng: np.random.Generator | None = None, name: str = "custom") -> LogitsVerifyInputs:
    """fp32 logits as given; drafts drawn from the tempered draft rows (input recipe only: the
    draft model's own sampling); open-interval uniforms."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    zp32 = np.ascontiguousarray(zp, dtype=np.float32)
    zq32 = np.ascontiguousarray(zq, dtype=np.float32)
    B, k1, V = zp32.shape
    k = k1 - 1
    temps = np.asarray(temps, dtype=np.float32).reshape(B)
    drafts = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):
            if temps[b] == 0:
                drafts[b, i] = int(np.argmax(zq32[b, i]))
            else:
                w = _softmax_rows_f64(zq32[b, i].astype(np.float64) / float(temps[b]))
                drafts[b, i] = rng.choice(V, p=w / w.sum())
    u = open_uniforms(rng, (B, k + 1))
    return LogitsVerifyInputs(name=name, seed=seed, zp=torch.from_numpy(zp32), zq=torch.from_numpy(zq32),
                              temps=torch.from_numpy(temps), draft_ids=torch.from_numpy(drafts),
                              uniforms=torch.from_numpy(u))


def logits_verify_config(name: str, seed: int | None = None, batch: int | None = None,
                         temps=None) -> LogitsVerifyInputs:
    """Named verification-from-logits workloads.

    tiny              B 4, k 4, V 1000; logits as verify_config("tiny"); temperatures cycle
                      through 1.0, 0.7, 0 (greedy), 1.3
    spec_verify_step  B 16, k 4, V 128256; logits as verify_config("spec_verify_step");
                      temperature 1 for every sequence
    ``batch`` overrides B, ``temps`` the temperatures.
    """
    if seed is None:
        seed = DEFAULT_SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny":
        B, k, V = batch or 4, 4, 1000
        pl = 2.0 * rng.standard_normal((B, k + 1, V))
        ql = 2.0 * rng.standard_normal((B, k, V))
        default = np.resize(np.array([1.0, 0.7, 0.0, 1.3]), B)
    elif name == "spec_verify_step":
        B, k, V = batch or 16, 4, 128256
        pl = 3.0 * rng.standard_normal((B, k + 1, V))
        ql = pl[:, :k] + 0.7 * rng.standard_normal((B, k, V))
        default = np.ones(B)
    else:
        raise KeyError(name)
    return make_logits_verify_inputs(seed, pl, ql, default if temps is None else temps, rng=rng, name=name)


# ----------------------------------------------------------------------------------------
# tree verification inputs
# ----------------------------------------------------------------------------------------

@dataclass
class TreeVerifyInputs:
    """One batch for verifying draft token trees (CPU tensors).

    p         fp32  [B, N, V]   target next-token distribution after each node
    q         fp32  [B, N, V]   draft distribution each node's children were drawn from
    parents   int32 [B, N]      parent of each node (-1 for the root, node 0); parents first
    tokens    int32 [B, N]      draft token of each node (entry 0, the root, unused: -1)
    uniforms  fp32  [B, N]      u[:, i] the accept test of node i > 0, u[:, 0] the final draw
    """

    name: str
    seed: int
    p: torch.Tensor
    q: torch.Tensor
    parents: torch.Tensor
    tokens: torch.Tensor
    uniforms: torch.Tensor

    @property
    def num_seqs(self) -> int:
        return int(self.p.shape[0])

    @property
    def num_nodes(self) -> int:
        return int(self.p.shape[1])

    @property
    def vocab(self) -> int:
        return int(self.p.shape[2])


def make_tree_verify_from_probs(seed: int, p32: np.ndarray, q32: np.ndarray, parents: np.ndarray,
                                rng: np.random.Generator | None = None, name: str = "custom") -> TreeVerifyInputs:
    """Children's tokens drawn independently from their parent's draft row, then uniforms."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    B, N, V = p32.shape
    parents = np.asarray(parents, dtype=np.int64).reshape(B, N)
    tokens = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        for i in range(1, N):
            w = q32[b, int(parents[b, i])].astype(np.float64)
            tokens[b, i] = rng.choice(V, p=w / w.sum())
    u = open_uniforms(rng, (B, N))
    return TreeVerifyInputs(name=name, seed=seed, p=torch.from_numpy(np.ascontiguousarray(p32)),
                            q=torch.from_numpy(np.ascontiguousarray(q32)),
                            parents=torch.from_numpy(parents.astype(np.int32)),
                            tokens=torch.from_numpy(tokens), uniforms=torch.from_numpy(u))


def tree_verify_config(name: str, seed: int | None = None, batch: int | None = None) -> TreeVerifyInputs:
    """Named tree-verification workloads (trees are random recursive trees, node 0 the root).

    tiny_tree         B 4, N 9, V 1000; target and draft logits independent N(0, 2)
    tree_verify_step  B 16, N 16, V 128256; target logits N(0, 3) per node; draft logits =
                      target logits + N(0, 0.7)
    """
    if seed is None:
        seed = DEFAULT_SEEDS.get(name, 2001)
    rng = np.random.Generator(np.random.PCG64(seed))
    if name == "tiny_tree":
        B, N, V = batch or 4, 9, 1000
        pl = 2.0 * rng.standard_normal((B, N, V))
        ql = 2.0 * rng.standard_normal((B, N, V))
    elif name == "tree_verify_step":
        B, N, V = batch or 16, 16, 128256
        pl = 3.0 * rng.standard_normal((B, N, V))
        ql = pl + 0.7 * rng.standard_normal((B, N, V))
    else:
        raise KeyError(name)
    parents = np.stack([random_tree_parents(rng, N) for _ in range(B)])
    p32 = _softmax_rows_f64(pl).astype(np.float32)
    q32 = _softmax_rows_f64(ql).astype(np.float32)
    return make_tree_verify_from_probs(seed, p32, q32, parents, rng=rng, name=name)
