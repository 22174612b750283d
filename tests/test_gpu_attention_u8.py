"""GPU parity of paged_attn_step_u8 (8-bit KV, dequantised in the kernel) against the oracle.

Same bar as the bf16 path: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise, the oracle
dequantising in float64, on every (row, head): the small cases and the full-size workloads
(same lengths and shapes as the bf16 ones, 8-bit codes) in the benchmark's launch
configuration; plus bitwise determinism and placement invariance.
"""

import numpy as np
import pytest
import torch

import verify_attention_paged_amd as vap
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _run(inp, workspace=None, scale=0.0):
    d = H.to_device(inp)
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                              scale=scale, workspace=workspace, kv_scales=d["kv_scales"])
    torch.cuda.synchronize()
    return out, d


def _case(seed, ctx, ql, Hq, Hkv, D, bs, **kw):
    return workloads.make_attention_inputs(seed, ctx_lens=ctx, q_lens=ql, num_q_heads=Hq, num_kv_heads=Hkv,
                                           head_dim=D, block_size=bs, kv_format="u8", **kw)


def test_tiny_config_full_parity():
    inp = H.config_inputs("tiny", "u8")
    print("tiny u8", inp.ctx_lens.tolist(), flush=True)
    out, _ = _run(inp)
    H.assert_close_rows(out, H.oracle_rows(inp), "tiny u8")


@pytest.mark.parametrize("name", ["llama3_8b_decode", "spec_verify_step", "llama70b_share", "mixed_step"])
def test_full_size_config_full_parity(name):
    inp = H.config_inputs(name, "u8")
    print(name, "u8: B", inp.num_seqs, "T", inp.total_q, "sum L", int(inp.ctx_lens.sum()), flush=True)
    ref = H.config_oracle(name, "u8")     # on the CPU, before the GPU call
    out, d = _run(inp)
    H.assert_full_parity(out, inp, ref, name + " u8")
    out2 = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                               kv_scales=d["kv_scales"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


FUZZ = [
    # (ctx_lens, q_lens, Hq, Hkv, D, bs)
    ([1, 2, 15, 16, 17, 31, 32, 33], [1] * 8, 8, 2, 64, 16),
    ([1, 2, 15, 16, 17, 31, 32, 33], [1] * 8, 4, 4, 128, 32),
    ([5, 16, 17, 40, 100], [5, 5, 5, 5, 5], 32, 8, 128, 16),
    ([5, 16, 17, 40, 100], [5, 2, 17, 1, 5], 32, 8, 128, 32),
    ([300, 7, 64, 65], [256, 7, 1, 17], 16, 2, 64, 16),
    ([1000, 3, 513], [1, 2, 3], 64, 8, 128, 16),
    ([2048, 1, 4096], [1, 1, 1], 8, 1, 128, 32),
    ([77, 78, 79], [1, 5, 1], 32, 32, 64, 16),
]


@pytest.mark.parametrize("case", range(len(FUZZ)))
def test_ragged_fuzz_full_parity(case):
    ctx, ql, Hq, Hkv, D, bs = FUZZ[case]
    print("fuzz u8", FUZZ[case], flush=True)
    inp = _case(300 + case, ctx, ql, Hq, Hkv, D, bs)
    out, _ = _run(inp)
    H.assert_close_rows(out, H.oracle_rows(inp), f"fuzz u8 {case}")


def test_block_placement_does_not_change_a_bit():
    """The same codes and scales in another pool placement give identical outputs."""
    inp = _case(11, np.array([17, 300, 64, 1000]), np.array([1, 5, 1, 5]), 32, 8, 128, 16)
    out, _ = _run(inp)
    NB = inp.num_blocks
    perm = np.random.default_rng(5).permutation(NB)         # new home of block b
    codes = torch.empty_like(inp.kv_pool)
    codes[:, torch.from_numpy(perm)] = inp.kv_pool
    scales = torch.empty_like(inp.kv_scales)
    scales[torch.from_numpy(perm)] = inp.kv_scales
    t = inp.block_tables.numpy()
    tables = torch.from_numpy(np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32))
    moved = workloads.AttnInputs(name="moved", seed=0, q=inp.q, kv_pool=codes, block_tables=tables,
                                 ctx_lens=inp.ctx_lens, q_lens=inp.q_lens, num_q_heads=inp.num_q_heads,
                                 num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                                 block_size=inp.block_size, kv_scales=scales)
    out2, _ = _run(moved)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("ws_kind", ["min", "small"])
def test_split_partition_invariance(ws_kind):
    inp = _case(12, [700, 33, 2100, 5], [1, 5, 1, 1], 32, 8, 128, 16)
    ref, d = _run(inp)
    shape = vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"])
    lib = vap.load_library()
    n = lib.vap_attn_workspace_min_bytes(__import__("ctypes").byref(shape))
    if ws_kind == "small":
        n = n * 40
    ws = torch.zeros(n, dtype=torch.uint8, device=d["q"].device)
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                              workspace=ws, kv_scales=d["kv_scales"])
    torch.cuda.synchronize()
    H.assert_close_rows(out, H.oracle_rows(inp), f"u8 {ws_kind} workspace")
    assert (out - ref).abs().max().item() < 1e-4


def test_bad_block_id_sets_error_without_fault():
    inp = _case(13, [40, 70], [1, 1], 8, 2, 64, 16)
    d = H.to_device(inp)
    bt = d["block_tables"].clone()
    bt[1, 2] = inp.num_blocks + 5
    ws = vap.attn_workspace(vap.attn_shape(d["q"], d["kv_pool"], bt), d["q"].device)
    out = vap.paged_attn_step(d["q"], d["kv_pool"], bt, d["ctx_lens"], d["q_lens"], workspace=ws,
                              kv_scales=d["kv_scales"])
    err = vap.get_device_error(ws)
    assert err & vap.DERR_BLOCK_ID
    # the unaffected sequence is still right
    ref = H.oracle_rows(inp, rows=[(0, h) for h in range(inp.num_q_heads)])
    H.assert_close_rows(out, ref, "u8 sequence 0 next to a bad block id")
