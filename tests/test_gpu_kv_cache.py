"""GPU parity of kv_append and kv_commit against the oracle (through the C ABI).

Bar: bit-exact.  Append copies bf16 rows or quantises them in fp32 with the same operations as
the oracle (IEEE division, round-half-even), so the whole pool, the codes and the scale words
(compared as bit patterns, poison included) must equal the oracle's.  Commit moves rows, so the
pool and the committed lengths must equal the oracle's exactly.
"""

import numpy as np
import pytest
import torch

import verify_attention_paged_amd as vap
import workloads
from oracle import attention as OA
from oracle import kv_cache as OK
from oracle import tree_verify as OT
from tests.gpu_helpers import assert_close_rows, bits, config_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inp(seed, L, Q, *, Hq=8, Hkv=2, D=64, bs=16, fmt="bf16"):
    return workloads.make_attention_inputs(seed, ctx_lens=L, q_lens=Q, num_q_heads=Hq, num_kv_heads=Hkv,
                                           head_dim=D, block_size=bs, kv_format=fmt)


def _dev(inp, tables=None, ctx=None, q=None):
    t = lambda x: torch.as_tensor(x).to(DEV).contiguous()
    pool = inp.kv_pool.to(DEV)
    sc = inp.kv_scales.to(DEV) if inp.kv_scales is not None else None
    return (pool, sc, t(inp.block_tables if tables is None else tables), t(inp.ctx_lens if ctx is None else ctx),
            t(inp.q_lens if q is None else q))


def _u32(x):
    return np.ascontiguousarray(x).view(np.uint32)


def _append_both(inp, k, v, oracle=True, **over):
    """Run kv_append on the GPU and in the oracle; return ((pool, scales) gpu, oracle)."""
    pool, sc, tables, ctx, ql = _dev(inp, **over)
    ws = vap.kv_workspace(DEV)
    vap.kv_append(k.to(DEV), v.to(DEV), pool, tables, ctx, ql, kv_scales=sc, workspace=ws)
    err = vap.get_device_error(ws)
    if not oracle:
        return (bits(pool.cpu()), None), None, err
    tab = tables.cpu().numpy()
    L, Q = ctx.cpu().numpy(), ql.cpu().numpy()
    if sc is None:
        ref = OK.kv_append(bits(inp.kv_pool), tab, L, Q, bits(k), bits(v))
        return (bits(pool.cpu()), None), (ref, None), err
    rc, rs = OK.kv_append_u8(inp.kv_pool.numpy(), inp.kv_scales.numpy(), tab, L, Q,
                             k.float().numpy(), v.float().numpy())
    return (pool.cpu().numpy(), sc.cpu().numpy()), (rc, rs), err


def _assert_same(got, ref, what):
    gp, gs = got
    rp, rs = ref
    bad = np.nonzero(gp != rp)
    assert bad[0].size == 0, f"{what}: {bad[0].size} pool entries differ, first at {tuple(int(b[0]) for b in bad)}"
    if rs is not None:
        badsc = np.nonzero(_u32(gs) != _u32(rs))
        assert badsc[0].size == 0, f"{what}: {badsc[0].size} scale words differ, first at {tuple(int(b[0]) for b in badsc)}"


@pytest.mark.parametrize("fmt", ["bf16", "u8"])
@pytest.mark.parametrize("D,bs", [(64, 16), (128, 16), (64, 32), (128, 32)])
def test_append_ragged_batch_bit_exact(fmt, D, bs):
    L, Q = [20, 64, 100, 33, 1, 300], [5, 1, 17, 33, 1, 64]
    inp = _inp(40 + D + bs, L, Q, Hkv=3 if D == 64 else 8, Hq=24 if D == 64 else 32, D=D, bs=bs, fmt=fmt)
    k, v = workloads.new_kv_rows(7, inp.total_q, inp.num_kv_heads, D)
    got, ref, err = _append_both(inp, k, v)
    assert err == 0
    _assert_same(got, ref, f"{fmt} D{D} bs{bs}")


@pytest.mark.parametrize("fmt", ["bf16", "u8"])
@pytest.mark.parametrize("name", ["llama3_8b_decode", "mixed_step", "tree_verify_step"])
def test_append_full_size_bit_exact(fmt, name):
    inp = config_inputs(name, fmt)
    k, v = workloads.new_kv_rows(11, inp.total_q, inp.num_kv_heads, inp.head_dim)
    got, ref, err = _append_both(inp, k, v)
    assert err == 0
    _assert_same(got, ref, f"{name} {fmt}")


@pytest.mark.parametrize("fmt", ["bf16", "u8"])
def test_append_above_the_staged_batch_limit(fmt):
    """More than 4096 sequences: the append kernel reads the lengths from global memory."""
    rng = np.random.default_rng(44)
    B = 5000
    Q = rng.integers(1, 4, size=B)
    L = np.maximum(Q, rng.integers(1, 80, size=B))
    inp = _inp(45, L, Q, Hq=4, Hkv=2, D=64, bs=16, fmt=fmt)
    k, v = workloads.new_kv_rows(46, inp.total_q, 2, 64)
    got, ref, err = _append_both(inp, k, v)
    assert err == 0
    _assert_same(got, ref, f"B {B} {fmt}")


def test_append_quantiser_edge_rows():
    """All-zero, constant, one-signed, single-outlier and tiny-range rows."""
    L, Q = [40, 9], [8, 9]
    inp = _inp(3, L, Q, Hkv=2, D=128, fmt="u8")
    k, v = workloads.new_kv_rows(5, inp.total_q, 2, 128)
    k, v = k.clone(), v.clone()
    k[0, 0] = 0.0
    k[1, 0] = 3.5
    k[2, 0] = -0.125
    k[3, 0] = k[3, 0].abs()
    k[4, 0] = -k[4, 0].abs()
    k[5, 0] = 0.0
    k[5, 0, 17] = 1000.0
    v[6, 1] = 1e-3 * torch.arange(128, dtype=torch.float32).to(torch.bfloat16)
    v[7, 1] = -65504.0
    v[8, 0, ::2] = 1e-30
    got, ref, err = _append_both(inp, k, v)
    assert err == 0
    _assert_same(got, ref, "edge rows")


def test_append_bad_rows_are_skipped_and_flagged():
    L, Q = [40, 50, 30], [4, 3, 6]
    inp = _inp(9, L, Q)
    k, v = workloads.new_kv_rows(2, inp.total_q, 2, 64)
    tables = inp.block_tables.clone()
    tables[1, 2] = inp.kv_pool.shape[1]          # the blocks of sequence 1's new rows (47, 48, 49)
    tables[1, 3] = inp.kv_pool.shape[1]
    got, ref, err = _append_both(inp, k, v, oracle=False, tables=tables)
    assert err & vap.DERR_BLOCK_ID
    # sequence 1 wrote nothing; the others match the oracle with sequence 1 left out
    keep = OK.kv_append(bits(inp.kv_pool), inp.block_tables.numpy()[[0, 2]], np.array(L)[[0, 2]],
                        np.array(Q)[[0, 2]], np.concatenate([bits(k)[:4], bits(k)[7:]]),
                        np.concatenate([bits(v)[:4], bits(v)[7:]]))
    _assert_same(got, (keep, None), "bad block id")
    ctx = inp.ctx_lens.clone()
    ctx[2] = 5                                                 # q_len 6 > ctx_len 5
    got, ref, err = _append_both(inp, k, v, oracle=False, ctx=ctx)
    assert err & vap.DERR_LENS
    keep = OK.kv_append(bits(inp.kv_pool), inp.block_tables.numpy()[:2], np.array(L)[:2], np.array(Q)[:2],
                        bits(k)[:7], bits(v)[:7])
    _assert_same(got, (keep, None), "q_len > ctx_len")


def test_append_total_q_mismatch_is_flagged():
    L, Q = [40, 50], [4, 3]
    inp = _inp(10, L, Q)
    k, v = workloads.new_kv_rows(3, 9, 2, 64)                 # total_q 9 > 7 rows the lengths cover
    got, ref, err = _append_both(inp, k, v)
    assert err & vap.DERR_TOTAL_Q
    _assert_same(got, ref, "extra rows ignored")


# ---------------------------------------------------------------------------------------------
# commit
# ---------------------------------------------------------------------------------------------

def _walk(parents, rng, max_len):
    """A root-to-node path through a tree (children chosen at random), as node indices."""
    kids = {}
    for c, p in enumerate(parents):
        kids.setdefault(int(p), []).append(c)
    path, u = [], 0
    while u in kids and len(path) < max_len:
        u = int(rng.choice(kids[u]))
        path.append(u)
    return path


def _commit_both(inp, path_rows, n, *, in_place=False, oracle=True, stride=None):
    pool, sc, tables, ctx, ql = _dev(inp)
    path = None
    if path_rows is not None:
        stride = stride or max(1, max(len(p) for p in path_rows) + 1)
        arr = np.full((len(path_rows), stride), -1, np.int32)
        for s, p in enumerate(path_rows):
            arr[s, :len(p)] = p
        path = torch.from_numpy(arr).to(DEV)
    n_t = torch.as_tensor(np.asarray(n, np.int32)).to(DEV)
    ws = vap.kv_workspace(DEV)
    out = vap.kv_commit(pool, tables, ctx, ql, n_t, path=path, kv_scales=sc,
                        out_ctx_lens=ctx if in_place else None, workspace=ws)
    err = vap.get_device_error(ws)
    if not oracle:
        return (bits(pool.cpu()), None), None, out.cpu().numpy(), None, err, ctx
    tab, L, Q = inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy()
    chain = [list(range(1, Q[s])) for s in range(len(L))]
    paths = path_rows if path_rows is not None else chain
    if sc is None:
        rp, _, rl = OK.kv_commit_tree(bits(inp.kv_pool), tab, L, Q, paths, n)
        got = (bits(pool.cpu()), None)
        ref = (rp, None)
    else:
        rp, rs, rl = OK.kv_commit_tree(inp.kv_pool.numpy(), tab, L, Q, paths, n, kv_scales=inp.kv_scales.numpy())
        got = (pool.cpu().numpy(), sc.cpu().numpy())
        ref = (rp, rs)
    return got, ref, out.cpu().numpy(), rl, err, ctx


@pytest.mark.parametrize("fmt", ["bf16", "u8"])
def test_tree_commit_bit_exact(fmt):
    rng = np.random.default_rng(21)
    sizes = [9, 16, 5, 64, 1, 33]
    L = [40, 100, 20, 300, 7, 64]
    parents = [workloads.random_tree_parents(rng, q) for q in sizes]
    # sequence 3: a caterpillar whose accepted path 2, 3, ..., 63 overlaps its destinations
    parents[3] = np.array([-1, 0, 0] + list(range(2, 63)))
    inp = _inp(22, L, sizes, Hq=32, Hkv=8, D=128, fmt=fmt)
    paths = [_walk(p, rng, 64) for p in parents]
    paths[3] = list(range(2, 64))
    n = [len(p) for p in paths]
    got, ref, lens, rl, err, _ = _commit_both(inp, paths, n)
    assert err == 0
    _assert_same(got, ref, f"tree commit {fmt}")
    assert np.array_equal(lens, rl)


def test_partial_acceptance_and_chain_commit_in_place():
    rng = np.random.default_rng(5)
    sizes = [9, 16, 5]
    inp = _inp(23, [40, 100, 20], sizes)
    parents = [workloads.random_tree_parents(rng, q) for q in sizes]
    full = [_walk(p, rng, 64) for p in parents]
    n = [min(len(p), c) for p, c in zip(full, (1, 2, 0))]     # a prefix of each walk accepted
    got, ref, lens, rl, err, _ = _commit_both(inp, full, n)
    assert err == 0
    _assert_same(got, ref, "partial paths")
    assert np.array_equal(lens, rl)
    # chain (no path): nothing moves, lengths updated in place
    n = [4, 0, 3]
    got, ref, lens, rl, err, ctx = _commit_both(inp, None, n, in_place=True)
    assert err == 0
    _assert_same(got, (bits(inp.kv_pool), None), "chain leaves the pool")
    assert np.array_equal(ctx.cpu().numpy(), rl) and np.array_equal(lens, rl)


def test_commit_errors_leave_the_sequence():
    sizes = [9, 6]
    inp = _inp(24, [40, 30], sizes)
    # n beyond q_len - 1
    got, ref, lens, rl, err, _ = _commit_both(inp, None, [9, 2], oracle=False)
    assert err & vap.DERR_LENS
    assert lens.tolist() == [40, int(30 - 6 + 1 + 2)]
    # a path that is not increasing: sequence 0 untouched, sequence 1 committed
    paths = [[3, 2], [1, 4]]
    got, ref, lens, rl, err, _ = _commit_both(inp, paths, [2, 2], oracle=False)
    assert err & vap.DERR_TREE
    assert lens.tolist() == [40, int(30 - 6 + 1 + 2)]
    rp, _, _ = OK.kv_commit_tree(bits(inp.kv_pool), inp.block_tables.numpy()[1:], inp.ctx_lens.numpy()[1:],
                                 inp.q_lens.numpy()[1:], paths[1:], [2])
    _assert_same(got, (rp, None), "bad path skipped")
    # n longer than the path rows: flagged, sequence left
    got, ref, lens, rl, err, _ = _commit_both(inp, [[1], [1]], [2, 1], oracle=False, stride=1)
    assert err & vap.DERR_TREE
    assert lens.tolist() == [40, int(30 - 6 + 1 + 1)]


# ---------------------------------------------------------------------------------------------
# one whole step: append, tree attention, tree verification, commit, next decode
# ---------------------------------------------------------------------------------------------

def _parents_from_masks(masks, sizes):
    out, t = [], 0
    for q in sizes:
        par = [-1]
        for i in range(1, q):
            m = int(masks[t + i]) & ((1 << i) - 1)
            par.append(m.bit_length() - 1)
        out.append(np.array(par))
        t += q
    return out


def test_step_append_verify_commit_then_decode():
    inp = config_inputs("tree_verify_step", "bf16")
    B, sizes = inp.num_seqs, inp.q_lens.numpy()
    masks = inp.tree_mask.numpy()
    parents = _parents_from_masks(masks, sizes)
    N = int(sizes.max())
    par = np.stack([np.concatenate([p, -np.ones(N - p.size, np.int64)]) for p in parents])
    # verifier inputs over the same trees (draft rows close to the target rows, so paths are long)
    rng = np.random.default_rng(77)
    V = 512
    soft = lambda z: np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True)
    pl = 3.0 * rng.standard_normal((B, N, V))
    p32 = soft(pl).astype(np.float32)
    q32 = soft(pl + 0.3 * rng.standard_normal((B, N, V))).astype(np.float32)
    tin = workloads.make_tree_verify_from_probs(78, p32, q32, par)
    u = OT.tree_uniforms_with_margin(p32, q32, par, tin.tokens.numpy(), tin.uniforms.numpy(), np.random.default_rng(79))
    ref_ids, ref_path, ref_n = OT.tree_verify(p32, q32, par, tin.tokens.numpy(), u.astype(np.float64))

    # GPU: append the step's rows, tree attention, verify, commit, decode the last accepted node
    k, v = workloads.new_kv_rows(80, inp.total_q, inp.num_kv_heads, inp.head_dim)
    pool, _, tables, ctx, ql = _dev(inp)
    ws = vap.attn_workspace(vap.attn_shape(inp.q.to(DEV), pool, tables), DEV)
    q = inp.q.to(DEV)
    vap.kv_append(k.to(DEV), v.to(DEV), pool, tables, ctx, ql, workspace=ws)
    tree_out = vap.paged_attn_step(q, pool, tables, ctx, ql, workspace=ws, tree_mask=inp.tree_mask.to(DEV))
    t = lambda x, dt: torch.as_tensor(np.ascontiguousarray(x, dtype=dt)).to(DEV)
    ids, path, n = vap.spec_verify_tree(t(p32, np.float32), t(q32, np.float32), t(par, np.int32),
                                        t(tin.tokens.numpy(), np.int32), t(u, np.float32))
    assert np.array_equal(path.cpu().numpy(), ref_path) and np.array_equal(n.cpu().numpy(), ref_n)
    new_L = vap.kv_commit(pool, tables, ctx, ql, n, path=path, workspace=ws)
    starts = np.concatenate([[0], np.cumsum(sizes)])
    last = np.array([ref_path[s][ref_n[s] - 1] if ref_n[s] else 0 for s in range(B)])
    rows = torch.as_tensor((starts[:-1] + last).astype(np.int64)).to(DEV)
    q_dec = q.index_select(0, rows).contiguous()
    dec = vap.paged_attn_step(q_dec, pool, tables, new_L, torch.ones(B, dtype=torch.int32, device=DEV), workspace=ws)
    assert vap.get_device_error(ws) == 0

    # oracle: the same step on the CPU
    pool1 = OK.kv_append(bits(inp.kv_pool), inp.block_tables.numpy(), inp.ctx_lens.numpy(), sizes, bits(k), bits(v))
    pool2, _, L2 = OK.kv_commit_tree(pool1, inp.block_tables.numpy(), inp.ctx_lens.numpy(), sizes, ref_path, ref_n)
    assert np.array_equal(new_L.cpu().numpy(), L2)
    assert np.array_equal(bits(pool.cpu()), pool2)
    hs = range(0, inp.num_q_heads, 5)
    ref_dec = OA.paged_attention_bf16(bits(q_dec.cpu()), pool2, inp.block_tables.numpy(), L2, np.ones(B, np.int64),
                                      rows=[(s, h) for s in range(B) for h in hs])
    assert_close_rows(dec, ref_dec, "decode after commit")
    # and the decode row equals the tree attention of that node (same keys, same values)
    ref_tree = {(s, h): ref_dec[(s, h)] for s in range(B) for h in hs}
    tree_rows = tree_out.index_select(0, rows)
    assert_close_rows(tree_rows, ref_tree, "tree attention of the accepted node")
