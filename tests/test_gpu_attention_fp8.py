"""GPU parity of paged_attn_step_fp8 (FP8 E4M3 KV, dequantised in the kernel) against the oracle.

Same bar as the bf16 path: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise, the oracle
decoding E4M3 from the format definition and dequantising in float64, on every (row, head):
the small cases, ragged fuzz shapes, nonzero zero points, and the full-size workloads (same
lengths and shapes as the bf16 ones, E4M3 codes) in the benchmark's launch configuration; plus
bitwise determinism and placement invariance.
"""

import numpy as np
import pytest
import torch

import verify_attention_paged_amd as vap
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _run(inp, workspace=None):
    d = H.to_device(inp)
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                              workspace=workspace, kv_scales=d["kv_scales"], fp8=True)
    torch.cuda.synchronize()
    return out, d


def _case(seed, ctx, ql, Hq, Hkv, D, bs, **kw):
    return workloads.make_attention_inputs(seed, ctx_lens=ctx, q_lens=ql, num_q_heads=Hq, num_kv_heads=Hkv,
                                           head_dim=D, block_size=bs, kv_format="fp8", **kw)


def test_tiny_config_full_parity():
    inp = H.config_inputs("tiny", "fp8")
    assert inp.kv_format == "fp8"
    out, _ = _run(inp)
    H.assert_full_parity(out, inp, H.oracle_rows(inp), "tiny fp8")


@pytest.mark.parametrize("name", ["llama3_8b_decode", "spec_verify_step", "llama70b_share", "mixed_step"])
def test_full_size_config_full_parity(name):
    inp = H.config_inputs(name, "fp8")
    print(name, "fp8: B", inp.num_seqs, "T", inp.total_q, "sum L", int(inp.ctx_lens.sum()), flush=True)
    ref = H.config_oracle(name, "fp8")     # on the CPU, before the GPU call
    out, d = _run(inp)
    H.assert_full_parity(out, inp, ref, name + " fp8")
    out2 = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                               kv_scales=d["kv_scales"], fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


FUZZ = [
    # (ctx_lens, q_lens, Hq, Hkv, D, bs)
    ([1, 2, 15, 16, 17, 31, 32, 33], [1] * 8, 8, 2, 64, 16),
    ([1, 2, 15, 16, 17, 31, 32, 33], [1] * 8, 4, 4, 128, 32),
    ([5, 16, 17, 40, 100], [5, 5, 5, 5, 5], 32, 8, 128, 16),
    ([300, 7, 64, 65], [256, 7, 1, 17], 16, 2, 64, 16),
    ([1000, 3, 513], [1, 2, 3], 64, 8, 128, 16),
    ([2048, 1, 4096], [1, 1, 1], 8, 1, 128, 32),
]


@pytest.mark.parametrize("case", range(len(FUZZ)))
def test_ragged_fuzz_full_parity(case):
    ctx, ql, Hq, Hkv, D, bs = FUZZ[case]
    print("fuzz fp8", FUZZ[case], flush=True)
    inp = _case(500 + case, ctx, ql, Hq, Hkv, D, bs)
    out, _ = _run(inp)
    H.assert_full_parity(out, inp, H.oracle_rows(inp), f"fuzz fp8 {case}")


def test_nonzero_zero_points_and_extreme_codes():
    """Zero points enter as scale * (e4m3 - zero); codes include the largest magnitudes (+-448),
    subnormals and signed zeros."""
    inp = _case(520, [40, 300, 77], [1, 5, 3], 16, 4, 128, 16)
    rng = np.random.default_rng(521)
    sc = inp.kv_scales.clone()
    live = torch.isfinite(sc)
    z = torch.from_numpy(rng.uniform(-2.0, 2.0, size=sc.shape).astype(np.float32))
    sc[..., 1] = torch.where(live[..., 1], z[..., 1], sc[..., 1])
    sc[..., 3] = torch.where(live[..., 3], z[..., 3], sc[..., 3])
    sc[..., 0] = torch.where(live[..., 0], sc[..., 0] * 0.01, sc[..., 0])   # keep scores moderate at +-448
    codes = inp.kv_pool.clone()
    special = torch.tensor([0x7E, 0xFE, 0x01, 0x81, 0x00, 0x80, 0x77, 0xF7], dtype=torch.uint8)
    pick = torch.from_numpy(rng.integers(0, codes.numel(), size=4000))
    codes.view(-1)[pick] = special[torch.from_numpy(rng.integers(0, special.numel(), size=4000))]
    mod = workloads.AttnInputs(**{**inp.__dict__, "kv_pool": codes, "kv_scales": sc})
    out, _ = _run(mod)
    H.assert_full_parity(out, mod, H.oracle_rows(mod), "fp8 zero points and extreme codes")


def test_block_placement_does_not_change_a_bit():
    inp = _case(530, np.array([17, 300, 64, 1000]), np.array([1, 5, 1, 5]), 32, 8, 128, 16)
    out, _ = _run(inp)
    perm = np.random.default_rng(6).permutation(inp.num_blocks)
    codes = torch.empty_like(inp.kv_pool)
    codes[:, torch.from_numpy(perm)] = inp.kv_pool
    scales = torch.empty_like(inp.kv_scales)
    scales[torch.from_numpy(perm)] = inp.kv_scales
    t = inp.block_tables.numpy()
    tables = torch.from_numpy(np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32))
    moved = workloads.AttnInputs(**{**inp.__dict__, "kv_pool": codes, "kv_scales": scales, "block_tables": tables})
    out2, _ = _run(moved)
    assert torch.equal(out, out2)
    H.assert_full_parity(out, inp, H.oracle_rows(inp), "fp8 placement")
