"""Pins of the oracle's FP8 (E4M3) KV path (CPU only).

* The E4M3 decode against a library routine: torch's float8_e4m3fn (OCP FP8) conversion to
  float64, on every one of the 256 codes, NaN included.
* Hand-worked codes from the format's definition (sign, 4-bit exponent with bias 7, 3-bit
  mantissa, subnormals at exponent 0, no infinities).
* Attention over an FP8 cache against the bf16 path (itself pinned to torch's SDPA): with
  power-of-two scales and zero points 0, every dequantised value is exactly representable in
  bf16, so both paths see identical float64 inputs and must agree bit for bit.
* The zero points enter as scale * (value - zero); block placement changes nothing; poisoned
  scales of unowned slots and rows past ctx_len are never read.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_e4m3_decode_matches_torch_on_every_code():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = A.e4m3_to_f64(np.arange(256))
    assert mine.dtype == np.float64
    assert np.array_equal(mine, ref, equal_nan=True)
    assert np.isnan(mine[[0x7F, 0xFF]]).all() and np.isfinite(np.delete(mine, [0x7F, 0xFF])).all()


@pytest.mark.parametrize("code, value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x30, 0.5), (0x7E, 448.0), (0x77, 240.0),
    (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x04, 2.0 ** -7),
    (0xB8, -1.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
])
def test_e4m3_hand_worked_codes(code, value):
    # e.g. 0x3C = 0 0111 100: exponent 7 - 7 = 0, mantissa 1 + 4/8 -> 1.5; 0x07: subnormal 7 * 2^-9
    assert A.e4m3_to_f64(np.array([code]))[0] == value


def test_negative_zero_code():
    v = A.e4m3_to_f64(np.array([0x80]))[0]
    assert v == 0.0 and np.signbit(v)


def test_dequantize_fp8_scale_and_zero():
    codes = np.array([[0x38, 0x40, 0xB8, 0x00]], dtype=np.uint8)        # 1, 2, -1, 0
    out = A.dequantize_fp8(codes, np.array([0.25]), np.array([0.5]))
    np.testing.assert_array_equal(out, [[0.125, 0.375, -0.375, -0.125]])


def exact_fp8_batch(seed, ctx_lens, q_lens, Hq, Hkv, D, bs):
    """An FP8 batch and a bf16 batch holding exactly the same values: torch's E4M3 codes of
    N(0, 1) draws, scaled by 2^-e (e in 0..3) per (plane, block, head, token), zero points 0."""
    base = workloads.make_attention_inputs(seed, ctx_lens=ctx_lens, q_lens=q_lens, num_q_heads=Hq,
                                           num_kv_heads=Hkv, head_dim=D, block_size=bs)
    rng = np.random.default_rng(seed + 91)
    NB = base.num_blocks
    x = torch.from_numpy(rng.standard_normal((2, NB, bs, Hkv, D)).astype(np.float32))
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    e4 = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s = np.exp2(-rng.integers(0, 4, size=(2, NB, bs, Hkv))).astype(np.float32)
    values = (s[..., None].astype(np.float64) * e4).astype(np.float32)
    pool = torch.from_numpy(values).to(torch.bfloat16)
    assert torch.equal(pool.float(), torch.from_numpy(values))          # bf16-exact
    scales = np.zeros((NB, Hkv, bs, 4), np.float32)
    scales[..., 0] = s[0].transpose(0, 2, 1)
    scales[..., 2] = s[1].transpose(0, 2, 1)
    return base, codes, scales, _bits(pool)


@pytest.mark.parametrize("case", [
    dict(ctx_lens=[1, 17, 40, 64], q_lens=[1, 1, 1, 1], Hq=8, Hkv=2, D=64, bs=16),
    dict(ctx_lens=[9, 33, 70], q_lens=[5, 5, 3], Hq=8, Hkv=4, D=32, bs=16),
    dict(ctx_lens=[100, 31], q_lens=[1, 8], Hq=6, Hkv=3, D=16, bs=32),
])
def test_fp8_attention_equals_bf16_attention_on_exact_values(case):
    base, codes, scales, pool_bits = exact_fp8_batch(6, case["ctx_lens"], case["q_lens"], case["Hq"],
                                                    case["Hkv"], case["D"], case["bs"])
    qb = _bits(base.q)
    args = (base.block_tables.numpy(), base.ctx_lens.numpy(), base.q_lens.numpy())
    r8 = A.paged_attention_fp8(qb, codes, scales, *args)
    r16 = A.paged_attention_bf16(qb, pool_bits, *args)
    assert r8.keys() == r16.keys()
    for key in r16:
        np.testing.assert_array_equal(r8[key], r16[key])


def test_fp8_block_placement_invariance():
    inp = workloads.attention_config("tiny", kv_format="fp8")
    qb = _bits(inp.q)
    codes, scales = inp.kv_pool.numpy(), inp.kv_scales.numpy()
    tables = inp.block_tables.numpy()
    ref = A.paged_attention_fp8(qb, codes, scales, tables, inp.ctx_lens.numpy(), inp.q_lens.numpy())
    perm = np.random.default_rng(4).permutation(inp.num_blocks)
    codes2 = np.empty_like(codes)
    scales2 = np.empty_like(scales)
    codes2[:, perm] = codes
    scales2[perm] = scales
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    out = A.paged_attention_fp8(qb, codes2, scales2, tables2, inp.ctx_lens.numpy(), inp.q_lens.numpy())
    for key in ref:
        np.testing.assert_array_equal(out[key], ref[key])


def test_fp8_poisoned_scales_are_never_read():
    inp = workloads.attention_config("tiny", kv_format="fp8")
    assert inp.kv_format == "fp8" and np.isnan(inp.kv_scales.numpy()).any()
    out = A.paged_attention_fp8(_bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(),
                                inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy())
    assert all(np.isfinite(v).all() for v in out.values())
