"""Pins of the oracle's 8-bit KV path (CPU only).

* Dequantisation against a library routine: torch's per-channel affine quint8 quantisation
  (``torch.quantize_per_channel(...).dequantize()``) implements value = scale * (code - zero)
  independently of the oracle.
* Attention over an 8-bit cache against the bf16 path (itself pinned to torch's SDPA): with
  power-of-two scales and integer offsets every dequantised value is exactly representable in
  bf16, so both paths see identical float64 inputs and must agree bit for bit.  The codes come
  from torch's quantiser, the scales are stored in the library's [NB, Hkv, bs, 4] layout.
* Block placement invariance: moving blocks (codes and scales together) changes nothing.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dequantize_matches_torch_per_channel_affine(seed):
    g = torch.Generator().manual_seed(seed)
    n, D = 400, 32
    s32 = torch.rand(n, generator=g) * 0.03 + 0.005          # fp32 scales
    z = torch.randint(0, 256, (n,), generator=g, dtype=torch.int64)
    x = torch.randn(n, D, generator=g) * 3.0                  # saturates some codes at 0 / 255
    qx = torch.quantize_per_channel(x, s32.double(), z, 0, torch.quint8)
    codes = qx.int_repr().numpy()
    assert codes.min() == 0 and codes.max() == 255
    ref = qx.dequantize().numpy()
    mine = A.dequantize_u8(codes, s32.numpy(), z.numpy().astype(np.float32))
    assert mine.dtype == np.float64
    np.testing.assert_array_equal(mine.astype(np.float32), ref)


def exact_u8_batch(seed, ctx_lens, q_lens, Hq, Hkv, D, bs):
    """An 8-bit batch and a bf16 batch holding exactly the same values.

    Values are s * n with s = 2^-e (e in 3..6) per (plane, block, head, token) and integer n in
    [-112, 112]; zero points are integers in [112, 143], so codes n + zero lie in [0, 255].
    Codes are produced by torch's per-channel quantiser.
    """
    base = workloads.make_attention_inputs(seed, ctx_lens=ctx_lens, q_lens=q_lens, num_q_heads=Hq,
                                           num_kv_heads=Hkv, head_dim=D, block_size=bs)
    rng = np.random.default_rng(seed + 77)
    NB = base.num_blocks
    chans = NB * bs * Hkv
    codes = np.empty((2, NB, bs, Hkv, D), np.uint8)
    values = np.empty((2, NB, bs, Hkv, D), np.float32)
    scales = np.empty((NB, Hkv, bs, 4), np.float32)
    for plane in range(2):
        s = np.exp2(-rng.integers(3, 7, size=chans)).astype(np.float32)
        z = rng.integers(112, 144, size=chans)
        n = rng.integers(-112, 113, size=(chans, D))
        v = torch.from_numpy((s[:, None].astype(np.float64) * n).astype(np.float32))
        qv = torch.quantize_per_channel(v, torch.from_numpy(s).double(), torch.from_numpy(z), 0, torch.quint8)
        c = qv.int_repr().numpy()
        assert np.array_equal(c.astype(np.int64), n + z[:, None])
        codes[plane] = c.reshape(NB, bs, Hkv, D)
        values[plane] = qv.dequantize().numpy().reshape(NB, bs, Hkv, D)
        # channel (block, row, head) -> scales[block, head, row]
        scales[:, :, :, 2 * plane] = s.reshape(NB, bs, Hkv).transpose(0, 2, 1)
        scales[:, :, :, 2 * plane + 1] = z.reshape(NB, bs, Hkv).transpose(0, 2, 1)
    pool = torch.from_numpy(values).to(torch.bfloat16)
    assert torch.equal(pool.float(), torch.from_numpy(values))   # bf16-exact
    return base, codes, scales, _bits(pool)


@pytest.mark.parametrize("case", [
    dict(ctx_lens=[1, 17, 40, 64], q_lens=[1, 1, 1, 1], Hq=8, Hkv=2, D=64, bs=16),
    dict(ctx_lens=[9, 33, 70], q_lens=[5, 5, 3], Hq=8, Hkv=4, D=32, bs=16),
    dict(ctx_lens=[100, 31], q_lens=[1, 8], Hq=6, Hkv=3, D=16, bs=32),
])
def test_u8_attention_equals_bf16_attention_on_exact_values(case):
    base, codes, scales, pool_bits = exact_u8_batch(5, case["ctx_lens"], case["q_lens"], case["Hq"],
                                                   case["Hkv"], case["D"], case["bs"])
    qb = _bits(base.q)
    args = (base.block_tables.numpy(), base.ctx_lens.numpy(), base.q_lens.numpy())
    r8 = A.paged_attention_u8(qb, codes, scales, *args)
    r16 = A.paged_attention_bf16(qb, pool_bits, *args)
    assert r8.keys() == r16.keys()
    for key in r16:
        np.testing.assert_array_equal(r8[key], r16[key])


def test_u8_block_placement_invariance():
    inp = workloads.attention_config("tiny", kv_format="u8")
    qb = _bits(inp.q)
    codes, scales = inp.kv_pool.numpy(), inp.kv_scales.numpy()
    tables = inp.block_tables.numpy()
    ref = A.paged_attention_u8(qb, codes, scales, tables, inp.ctx_lens.numpy(), inp.q_lens.numpy())
    perm = np.random.default_rng(3).permutation(inp.num_blocks)     # new home of block b
    codes2 = np.empty_like(codes)
    scales2 = np.empty_like(scales)
    codes2[:, perm] = codes
    scales2[perm] = scales
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    out = A.paged_attention_u8(qb, codes2, scales2, tables2, inp.ctx_lens.numpy(), inp.q_lens.numpy())
    for key in ref:
        np.testing.assert_array_equal(out[key], ref[key])


def test_u8_poisoned_scales_are_never_read():
    """Scales of unowned slots and of rows past ctx_len are NaN; every output is finite."""
    inp = workloads.attention_config("tiny", kv_format="u8")
    assert np.isnan(inp.kv_scales.numpy()).any()
    out = A.paged_attention_u8(_bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(),
                               inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy())
    assert all(np.isfinite(v).all() for v in out.values())
