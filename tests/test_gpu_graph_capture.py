"""Whole steps captured in HIP graphs (torch.cuda.CUDAGraph) replay bit for bit like eager calls.

The library launches its kernels on the caller's stream, allocates nothing inside a call and
clears no memory with memset nodes, so a step (paged_attn_step, then spec_verify or
spec_verify_tree) can be captured once and replayed.  State that kernels keep in a workspace
between calls (arrival tickets, descriptors) returns to its start state within every call.
Each replay's outputs are cleared first, so a replay that did nothing fails; replays are
interleaved with eager calls of the library on other inputs and with synchronisations.
"""

import pytest
import torch

import verify_attention_paged_amd as vap
import workloads
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                               # one eager call on the side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _attention_args(name):
    inp = H.config_inputs(name)
    d = H.to_device(inp)
    if inp.tree_mask is not None:
        d["tree_mask"] = inp.tree_mask.to(H.device())
    return inp, d


def _eager_noise():
    """Eager library work between replays (another shape, its own workspace)."""
    inp = H.config_inputs("tiny")
    d = H.to_device(inp)
    return vap.paged_attn_step(**d)


def test_verify_step_graph_replays_match_eager():
    inp, d = _attention_args("spec_verify_step")
    ver = workloads.verify_config("spec_verify_step")
    dev = H.device()
    p, q = ver.p.to(dev), ver.q.to(dev)
    ids, uni = ver.draft_ids.to(dev), ver.uniforms.to(dev)
    out = torch.empty((inp.total_q, inp.num_q_heads, inp.head_dim), dtype=torch.float32, device=dev)
    out_ids = torch.empty((ver.num_seqs, ver.k + 1), dtype=torch.int32, device=dev)
    n_acc = torch.empty((ver.num_seqs,), dtype=torch.int32, device=dev)
    aws = vap.attn_workspace(vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"]), dev)
    sws = vap.verify_workspace(ver.num_seqs, ver.k, ver.vocab, dev)

    def step():
        vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"], out=out,
                            workspace=aws)
        vap.spec_verify(p, q, ids, uni, out_ids, n_acc, workspace=sws)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), out_ids.clone(), n_acc.clone())
    g = _capture(step)
    for r in range(3):
        print("verify step replay", r, flush=True)
        out.zero_()
        out_ids.fill_(-7)
        n_acc.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(out_ids, ref[1]) and torch.equal(n_acc, ref[2]), r
        _eager_noise()
        step()                             # eager calls on the same workspaces between replays
        torch.cuda.synchronize()
        assert torch.equal(out_ids, ref[1])
    assert vap.get_device_error(aws) == 0 and vap.get_device_error(sws) == 0


def test_tree_step_graph_replays_match_eager():
    inp, d = _attention_args("tree_verify_step")
    tver = workloads.tree_verify_config("tree_verify_step")
    dev = H.device()
    p, q = tver.p.to(dev), tver.q.to(dev)
    par, tok, uni = tver.parents.to(dev), tver.tokens.to(dev), tver.uniforms.to(dev)
    out = torch.empty((inp.total_q, inp.num_q_heads, inp.head_dim), dtype=torch.float32, device=dev)
    ids = torch.empty((tver.num_seqs, tver.num_nodes), dtype=torch.int32, device=dev)
    path = torch.empty_like(ids)
    n = torch.empty((tver.num_seqs,), dtype=torch.int32, device=dev)
    aws = vap.attn_workspace(vap.attn_shape(d["q"], d["kv_pool"], d["block_tables"]), dev)
    tws = vap.tree_verify_workspace(tver.num_seqs, dev)

    def step():
        vap.paged_attn_step(d["q"], d["kv_pool"], d["block_tables"], d["ctx_lens"], d["q_lens"], out=out,
                            workspace=aws, tree_mask=d["tree_mask"])
        vap.spec_verify_tree(p, q, par, tok, uni, ids, path, n, workspace=tws)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), ids.clone(), path.clone(), n.clone())
    g = _capture(step)
    for r in range(3):
        print("tree step replay", r, flush=True)
        out.zero_()
        ids.fill_(-7)
        path.fill_(-7)
        n.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = (out, ids, path, n)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), r
        _eager_noise()
        step()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref[1]) and torch.equal(n, ref[3])
    assert vap.get_device_error(aws) == 0 and vap.get_device_error(tws) == 0
