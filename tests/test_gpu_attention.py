"""GPU parity of paged_attn_step against the fp64 oracle (through the C ABI).

Bar: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise, on every (row, head) of every case:
the small cases, the full-size workloads in the launch configuration the benchmark uses, and
the batches above 2048 sequences; plus bitwise determinism and invariance to block placement.
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
                              scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return out, d


def _case(seed, ctx, ql, Hq, Hkv, D, bs, **kw):
    return workloads.make_attention_inputs(seed, ctx_lens=ctx, q_lens=ql, num_q_heads=Hq,
                                           num_kv_heads=Hkv, head_dim=D, block_size=bs, **kw)


def test_tiny_config_full_parity():
    inp = H.config_inputs("tiny")
    print("tiny", inp.ctx_lens.tolist(), flush=True)
    out, _ = _run(inp)
    H.assert_close_rows(out, H.oracle_rows(inp), "tiny")


@pytest.mark.parametrize("name", ["llama3_8b_decode", "spec_verify_step", "llama70b_share", "mixed_step"])
def test_full_size_config_full_parity(name):
    """Every (row, head) of the full-size workload, in the launch configuration the benchmark
    uses (default workspace), against the oracle element by element."""
    inp = H.config_inputs(name)
    print(name, "B", inp.num_seqs, "T", inp.total_q, "sum L", int(inp.ctx_lens.sum()), flush=True)
    ref = H.config_oracle(name)           # on the CPU, before the GPU call
    out, d = _run(inp)
    H.assert_full_parity(out, inp, ref, name)
    # a second call on the same inputs is bitwise identical (fixed reduction order)
    out2 = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"])
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
    ([33, 64], [33, 1], 8, 8, 128, 32),
]


@pytest.mark.parametrize("case", range(len(FUZZ)))
def test_ragged_fuzz_full_parity(case):
    ctx, ql, Hq, Hkv, D, bs = FUZZ[case]
    print("fuzz", FUZZ[case], flush=True)
    inp = _case(100 + case, ctx, ql, Hq, Hkv, D, bs)
    out, _ = _run(inp)
    H.assert_close_rows(out, H.oracle_rows(inp), f"fuzz {case}")


WIDE = [
    # batches averaging >= 48 rows per KV head and sequence run 64-row units (four row tiles);
    # (ctx_lens, q_lens, Hq, Hkv, D, bs, kv_format)
    ([40, 100, 20, 300], [16, 16, 16, 16], 32, 8, 128, 16, "bf16"),     # 64 rows per KV head
    ([1500, 3000, 64], [64, 17, 64], 16, 2, 64, 32, "bf16"),            # long contexts: 64-row partials
    ([4096, 900], [48, 48], 8, 8, 128, 16, "bf16"),                     # 48 rows (12 quads) per unit
    ([700, 33], [33, 33], 16, 4, 128, 32, "bf16"),                      # 132 rows: units 64, 64, 4
    ([2500, 70, 200], [64, 64, 17], 32, 8, 128, 16, "u8"),              # 8-bit cache
]


@pytest.mark.parametrize("case", range(len(WIDE)))
def test_wide_units_full_parity(case):
    ctx, ql, Hq, Hkv, D, bs, fmt = WIDE[case]
    print("wide", WIDE[case], flush=True)
    inp = _case(300 + case, ctx, ql, Hq, Hkv, D, bs, kv_format=fmt)
    d = H.to_device(inp)
    out = vap.paged_attn_step(**d)
    torch.cuda.synchronize()
    H.assert_close_rows(out, H.oracle_rows(inp), f"wide {case}")


def test_wide_units_with_the_minimum_workspace():
    """64-row units split over few worker waves: long partial lists of 64 rows each."""
    inp = _case(310, [4096, 2000, 80], [64, 64, 64], 32, 8, 128, 16)
    shape = vap.attn_shape(inp.q, inp.kv_pool, inp.block_tables)
    import ctypes
    lo = vap.load_library().vap_attn_workspace_min_bytes(ctypes.byref(shape))
    ws = torch.zeros(lo, dtype=torch.uint8, device=H.device())
    out, _ = _run(inp, workspace=ws)
    H.assert_close_rows(out, H.oracle_rows(inp), "wide, minimum workspace")


LARGE = [
    # batches above 2048 sequences take their plan from the plan kernel instead of LDS;
    # (batch, max ctx_len, max q_len, Hq, Hkv, D, bs, kv_format)
    (2049, 300, 5, 4, 1, 128, 16, "bf16"),
    (3000, 200, 1, 8, 2, 64, 16, "bf16"),
    (3000, 200, 3, 8, 2, 64, 32, "u8"),
    (8192, 40, 1, 2, 1, 64, 16, "bf16"),
]


@pytest.mark.parametrize("case", range(len(LARGE)))
def test_plan_kernel_path_large_batches(case):
    B, Lmax, Qmax, Hq, Hkv, D, bs, fmt = LARGE[case]
    print("large batch", LARGE[case], flush=True)
    rng = np.random.default_rng(900 + case)
    Q = rng.integers(1, Qmax + 1, size=B)
    L = np.maximum(Q, rng.integers(1, Lmax + 1, size=B))
    inp = _case(900 + case, L, Q, Hq, Hkv, D, bs, kv_format=fmt)
    d = H.to_device(inp)
    shape = vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"])
    ws = vap.attn_workspace(shape, H.device())
    out = vap.paged_attn_step(**d, workspace=ws)
    torch.cuda.synchronize()
    assert vap.get_device_error(ws) == 0
    H.assert_full_parity(out, inp, H.oracle_rows(inp), f"large {case}")


def test_block_placement_does_not_change_a_bit():
    """Same logical KV, two different pool permutations and pool sizes -> identical outputs."""
    ctx, ql = np.array([17, 300, 64, 1000]), np.array([1, 5, 1, 5])
    a = _case(7, ctx, ql, 32, 8, 128, 16)
    # rebuild the same logical K/V under a different placement
    rng = np.random.default_rng(99)
    NB = a.num_blocks + 13
    pool = torch.full((2, NB, 16, 8, 128), float("nan"), dtype=torch.bfloat16)
    tables = torch.full_like(a.block_tables, -1)
    perm = torch.from_numpy(rng.permutation(NB))
    c = 0
    for s in range(len(ctx)):
        nb = (int(ctx[s]) + 15) // 16
        for j in range(nb):
            src = int(a.block_tables[s, j])
            dst = int(perm[c])
            c += 1
            tables[s, j] = dst
            pool[:, dst] = a.kv_pool[:, src]
    b = workloads.AttnInputs(**{**a.__dict__, "kv_pool": pool, "block_tables": tables})
    out_a, _ = _run(a)
    out_b, _ = _run(b)
    assert torch.equal(out_a, out_b)
    H.assert_close_rows(out_a, H.oracle_rows(a), "placement")


def test_shared_prefix_blocks():
    """Two sequences whose tables share physical prefix blocks, same query -> same output."""
    inp = _case(8, [100, 100, 90], [1, 1, 1], 8, 2, 64, 16)
    tables = inp.block_tables.clone()
    tables[1, :4] = tables[0, :4]          # first 64 tokens shared
    tables[1, 4:7] = tables[0, 4:7]        # and the rest too: sequence 1 == sequence 0
    q = inp.q.clone()
    q[1] = q[0]
    shared = workloads.AttnInputs(**{**inp.__dict__, "block_tables": tables, "q": q})
    out, _ = _run(shared)
    assert torch.equal(out[0], out[1])
    H.assert_close_rows(out, H.oracle_rows(shared), "shared prefix")


@pytest.mark.parametrize("ws_kind", ["min", "small", "default"])
def test_split_partition_invariance(ws_kind):
    """Fewer worker waves (smaller workspace) change the split points, not the result."""
    inp = _case(9, [4096, 17, 1500, 33, 800, 2], [1, 5, 1, 2, 5, 1], 32, 8, 128, 16)
    shape = vap.attn_shape(inp.q, inp.kv_pool, inp.block_tables)
    lib = vap.load_library()
    import ctypes
    lo = lib.vap_attn_workspace_min_bytes(ctypes.byref(shape))
    hi = lib.vap_attn_workspace_bytes(ctypes.byref(shape))
    nbytes = {"min": lo, "small": (lo + hi) // 7 // 256 * 256, "default": hi}[ws_kind]
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=H.device())
    out, _ = _run(inp, workspace=ws)
    H.assert_close_rows(out, H.oracle_rows(inp), f"split {ws_kind}")


def test_one_workspace_across_calls_and_shapes():
    """Each call leaves the workspace ready for the next: repeated calls, and calls of other
    shapes, on one workspace give bitwise the results of calls on fresh workspaces."""
    import ctypes
    cases = {"decode": H.config_inputs("llama3_8b_decode"),
             "small": _case(21, [4096, 17, 1500, 33, 800, 2], [1, 5, 1, 2, 5, 1], 32, 8, 128, 16),
             "mixed": H.config_inputs("mixed_step")}
    lib = vap.load_library()
    nbytes = max(lib.vap_attn_workspace_bytes(ctypes.byref(vap.attn_shape(i.q, i.kv_pool, i.block_tables)))
                 for i in cases.values())
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=H.device())
    ref = {}
    for name, inp in cases.items():
        ref[name], _ = _run(inp)
    for name in ["decode", "small", "decode", "mixed", "decode", "small", "mixed"]:
        print("shared workspace:", name, flush=True)
        out, _ = _run(cases[name], workspace=ws)
        assert torch.equal(out, ref[name]), name
    assert vap.get_device_error(ws) == 0


@pytest.mark.parametrize("G, D, bs", [(4, 128, 16), (8, 128, 16), (4, 64, 32), (8, 128, 32)])
@pytest.mark.parametrize("ws_kind", ["min", "small"])
def test_pool_of_tail_pieces_full_parity(G, D, bs, ws_kind):
    """Decode batches on small workspaces (few worker waves) have far more than 32 work blocks per
    wave, so the last tenth of their work runs as pool pieces that finished waves claim: full
    parity with the oracle, bitwise-equal reruns on the same workspace, no device error."""
    import ctypes
    inp = _case(31 + G + D + bs, [3000, 17, 1500, 33, 800, 2, 640, 129, 2048, 4000], [1] * 10, 2 * G, 2, D, bs)
    shape = vap.attn_shape(inp.q, inp.kv_pool, inp.block_tables)
    lib = vap.load_library()
    lo = lib.vap_attn_workspace_min_bytes(ctypes.byref(shape))
    hi = lib.vap_attn_workspace_bytes(ctypes.byref(shape))
    nbytes = {"min": lo, "small": (lo + hi) // 9 // 256 * 256}[ws_kind]
    ws = torch.zeros(max(lo, nbytes), dtype=torch.uint8, device=H.device())
    print("pool case G", G, "D", D, "bs", bs, ws_kind, "workspace", ws.numel(), flush=True)
    out, d = _run(inp, workspace=ws)
    H.assert_close_rows(out, H.oracle_rows(inp), f"pool G={G} D={D} bs={bs} {ws_kind}")
    for _ in range(2):
        again = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                                    workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, again)
    assert vap.get_device_error(ws) == 0


def test_explicit_scale():
    inp = _case(10, [50, 200], [5, 1], 8, 2, 64, 16)
    out, _ = _run(inp, scale=0.3)
    H.assert_close_rows(out, H.oracle_rows(inp, scale=0.3), "scale 0.3")


def test_verify_rows_equal_decode_calls():
    """Row i of a q_len=5 call matches a q_len=1 call over the first L-(4-i) keys."""
    inp = _case(11, [700], [5], 32, 8, 128, 16)
    out, d = _run(inp)
    for i in range(5):
        dec_ctx = d["ctx_lens"] - (4 - i)
        one = vap.paged_attn_step(d["q"][i:i + 1].contiguous(), d["kv_pool"], d["block_tables"], dec_ctx,
                                  torch.ones_like(d["q_lens"]))
        torch.cuda.synchronize()
        diff = (one[0] - out[i]).abs().max().item()
        assert diff <= 1e-5, (i, diff)


def test_bad_block_id_sets_error_without_fault():
    inp = _case(12, [40, 40], [1, 1], 8, 2, 64, 16)
    d = H.to_device(inp)
    d["block_tables"][1, 1] = inp.num_blocks + 1000     # outside the pool
    ws = vap.attn_workspace(vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"]), H.device())
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"], workspace=ws)
    err = vap.get_device_error(ws, clear=True)
    assert err & vap.DERR_BLOCK_ID
    H.assert_close_rows(out[:1], {k: v for k, v in H.oracle_rows(inp).items() if k[0] == 0}, "untouched seq")
    assert vap.get_device_error(ws) == 0


def test_bad_block_id_deep_in_a_long_context_is_reported():
    """The error is flagged whichever lane of a wave reads the bad table entry."""
    inp = _case(14, [2000, 900], [1, 1], 8, 2, 64, 16)
    d = H.to_device(inp)
    d["block_tables"][0, 77] = -3                       # negative: outside the pool
    ws = vap.attn_workspace(vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"]), H.device())
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"], workspace=ws)
    assert vap.get_device_error(ws, clear=True) & vap.DERR_BLOCK_ID
    H.assert_close_rows(out[1:], {(t - 1, h): v for (t, h), v in H.oracle_rows(inp).items() if t == 1},
                        "untouched seq")


def test_bad_lengths_set_error_and_spare_other_sequences():
    inp = _case(13, [40, 40, 40], [1, 1, 1], 8, 2, 64, 16)
    d = H.to_device(inp)
    ref = H.oracle_rows(inp)
    d["q_lens"][1] = 41                                   # q_len > ctx_len
    ws = vap.attn_workspace(vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"]), H.device())
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"], workspace=ws)
    err = vap.get_device_error(ws, clear=True)
    assert err & vap.DERR_LENS
    H.assert_close_rows(out, {k: v for k, v in ref.items() if k[0] == 0}, "seq 0")
    d["q_lens"][1] = 1
    d["ctx_lens"][2] = 16 * inp.max_blocks_per_seq + 1    # beyond the table's capacity
    vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"], out=out, workspace=ws)
    assert vap.get_device_error(ws, clear=True) & vap.DERR_LENS
    H.assert_close_rows(out, {k: v for k, v in ref.items() if k[0] < 2}, "seqs 0-1")


def test_empty_batch_is_a_no_op():
    dev = H.device()
    q = torch.zeros(0, 8, 64, dtype=torch.bfloat16, device=dev)
    pool = torch.zeros(2, 1, 16, 2, 64, dtype=torch.bfloat16, device=dev)
    tables = torch.zeros(0, 1, dtype=torch.int32, device=dev)
    lens = torch.zeros(0, dtype=torch.int32, device=dev)
    out = vap.paged_attn_step(q, pool, tables, lens, lens)
    assert out.shape == (0, 8, 64)
