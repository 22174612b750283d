"""GPU parity of paged_attn_step_tree (tree-masked verify attention) against the oracle.

Bar as for the causal path: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise.  The oracle's
tree path is pinned to the causal verify (chains and root-to-node paths) on the CPU.
"""

import numpy as np
import pytest
import torch

import verify_attention_paged_amd as vap
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _tree_case(seed, ctx, Hq, Hkv, D, bs, sizes, kv_format="bf16"):
    rng = np.random.default_rng(seed)
    inp = workloads.make_attention_inputs(seed, ctx_lens=ctx, q_lens=sizes, num_q_heads=Hq, num_kv_heads=Hkv,
                                          head_dim=D, block_size=bs, kv_format=kv_format)
    inp.tree_mask = torch.from_numpy(np.concatenate(
        [workloads.tree_masks(workloads.random_tree_parents(rng, int(n))) for n in sizes]))
    return inp


def _run(inp, workspace=None):
    d = H.to_device(inp)
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                              workspace=workspace, kv_scales=d.get("kv_scales"),
                              tree_mask=inp.tree_mask.to(d["q"].device))
    torch.cuda.synchronize()
    return out, d


def _oracle(inp, rows=None):
    from oracle import attention as OA
    args = (inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy())
    if inp.kv_scales is not None:
        return OA.paged_attention_u8(H.bits(inp.q), inp.kv_pool.numpy(), inp.kv_scales.numpy(), *args,
                                     rows=rows, tree_mask=inp.tree_mask.numpy())
    return OA.paged_attention_bf16(H.bits(inp.q), H.bits(inp.kv_pool), *args, rows=rows,
                                   tree_mask=inp.tree_mask.numpy())


@pytest.mark.parametrize("kv_format", ["bf16", "u8"])
def test_tree_verify_step_full_parity(kv_format):
    inp = H.config_inputs("tree_verify_step", kv_format)
    print("tree_verify_step", kv_format, "T", inp.total_q, flush=True)
    ref = H.config_oracle("tree_verify_step", kv_format)   # on the CPU, before the GPU call
    out, d = _run(inp)
    H.assert_full_parity(out, inp, ref, f"tree_verify_step {kv_format}")


FUZZ = [
    # (ctx_lens, tree sizes, Hq, Hkv, D, bs)
    ([20, 64, 100, 300], [20, 9, 64, 33], 8, 2, 64, 16),
    ([17, 45, 1000], [1, 45, 16], 32, 8, 128, 16),        # no prefix for the 45-node tree
    ([500, 33, 2048], [24, 32, 60], 16, 4, 128, 32),
    ([70, 71], [64, 2], 8, 8, 64, 32),
]


@pytest.mark.parametrize("case", range(len(FUZZ)))
@pytest.mark.parametrize("kv_format", ["bf16", "u8"])
def test_random_trees_full_parity(case, kv_format):
    ctx, sizes, Hq, Hkv, D, bs = FUZZ[case]
    print("tree fuzz", kv_format, FUZZ[case], flush=True)
    inp = _tree_case(400 + case, ctx, Hq, Hkv, D, bs, sizes, kv_format)
    out, d = _run(inp)
    H.assert_close_rows(out, _oracle(inp), f"tree fuzz {case} {kv_format}")


def test_small_trees_with_the_pool_of_tail_pieces():
    """Trees of up to 4 nodes at G = 4 make 16-row units; on the minimum workspace (few worker
    waves, far more than 32 work blocks each) the last tenth of the work runs as pool pieces, so
    ranges start and end inside masked units: full parity, bitwise-equal rerun, no error."""
    import ctypes
    inp = _tree_case(470, [3000, 1500, 4000, 800, 2048, 129, 640, 17], 8, 2, 128, 16,
                     [4, 3, 2, 4, 1, 3, 4, 2])
    shape = vap.attn_shape(inp.q, inp.kv_pool, inp.block_tables)
    lo = vap.load_library().vap_attn_workspace_min_bytes(ctypes.byref(shape))
    ws = torch.zeros(lo, dtype=torch.uint8, device=H.device())
    out, d = _run(inp, workspace=ws)
    H.assert_close_rows(out, _oracle(inp), "small trees, pool")
    again, _ = _run(inp, workspace=ws)
    assert torch.equal(out, again)
    assert vap.get_device_error(ws) == 0


def test_chain_masks_match_the_causal_kernel():
    inp = workloads.make_attention_inputs(21, ctx_lens=[40, 300, 1000], q_lens=[5, 17, 64], num_q_heads=32,
                                          num_kv_heads=8, head_dim=128, block_size=16)
    d = H.to_device(inp)
    causal = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"])
    chain = torch.from_numpy(np.concatenate([workloads.tree_masks(np.arange(n) - 1) for n in (5, 17, 64)]))
    tree = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                               tree_mask=chain.to(d["q"].device))
    torch.cuda.synchronize()
    assert (tree - causal).abs().max().item() <= 1e-5
    H.assert_close_rows(tree, H.oracle_rows(inp), "chain masks")


def test_invalid_masks_set_the_error_bit_and_are_repaired():
    inp = _tree_case(31, [50, 60], 8, 2, 64, 16, [6, 8])
    m = inp.tree_mask.numpy().view(np.uint64).copy()
    m[2] &= ~np.uint64(1 << 2)              # node 2 of sequence 0 without its own bit
    m[6 + 3] |= np.uint64(1 << 7)           # node 3 of sequence 1 with a later node
    bad = torch.from_numpy(m.view(np.int64))
    repaired = m.copy()
    repaired[2] |= np.uint64(1 << 2)
    repaired[6 + 3] &= ~np.uint64(1 << 7)
    d = H.to_device(inp)
    ws = vap.attn_workspace(vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"]), H.device())
    out = vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"],
                              workspace=ws, tree_mask=bad.to(d["q"].device))
    assert vap.get_device_error(ws, clear=True) & vap.DERR_TREE
    inp.tree_mask = torch.from_numpy(repaired.view(np.int64))
    H.assert_close_rows(out, _oracle(inp), "repaired masks")
