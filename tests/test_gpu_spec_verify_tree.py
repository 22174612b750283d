"""GPU parity of spec_verify_tree against the sequential fp64 oracle (through the C ABI).

Bar: accepted counts, accepted node paths and token ids bit-exact, with uniforms placed at
least 1e-6 from every threshold the oracle's walk evaluates
(oracle.tree_verify.tree_uniforms_with_margin).  A Monte Carlo test with raw uniforms checks the
emitted distribution of the GPU walk directly.
"""

import json
import os

import numpy as np
import pytest
import torch
from scipy import stats

import verify_attention_paged_amd as vap
import workloads
from oracle import spec_verify as OS
from oracle import tree_verify as OT

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _t(x, dt):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=dt), device=DEV)


def _gpu(p, q, parents, tokens, u, workspace=None):
    out, path, n = vap.spec_verify_tree(_t(p, np.float32), _t(q, np.float32), _t(parents, np.int32),
                                        _t(tokens, np.int32), _t(u, np.float32), workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy(), path.cpu().numpy(), n.cpu().numpy()


def _compare(p, q, parents, tokens, u, what):
    ref = OT.tree_verify(p, q, parents, tokens, u.astype(np.float64))
    got = _gpu(p, q, parents, tokens, u)
    for name, a, b in zip(("ids", "path", "n_accepted"), got, ref):
        assert np.array_equal(a, b), f"{what}: {name} differ\n{a}\n{b}"
    return ref[2]


def _margin(tin, seed):
    p = tin.p.numpy()
    q = tin.q.numpy()
    u = OT.tree_uniforms_with_margin(p, q, tin.parents.numpy(), tin.tokens.numpy(), tin.uniforms.numpy(),
                                     np.random.default_rng(seed))
    return p, q, tin.parents.numpy(), tin.tokens.numpy(), u


def test_tiny_tree_bit_exact():
    _compare(*_margin(workloads.tree_verify_config("tiny_tree"), 1), "tiny_tree")


@pytest.mark.parametrize("seed", range(4))
def test_tiny_tree_recipe_many_seeds(seed):
    tin = workloads.tree_verify_config("tiny_tree", seed=3000 + seed, batch=24)
    _compare(*_margin(tin, seed), f"tiny_tree seed {seed}")


def test_tree_verify_step_full_size_bit_exact():
    tin = workloads.tree_verify_config("tree_verify_step")
    n = _compare(*_margin(tin, 2), "tree_verify_step")
    print("accepted per sequence", n.tolist(), flush=True)


def test_golden_cases_on_gpu():
    with open(os.path.join(GOLDEN, "tree_verify_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p = np.array(c["p"], np.float32)[None]
        q = np.array(c["q"], np.float32)[None]
        out, path, n = _gpu(p, q, np.array(c["parents"])[None], np.array(c["tokens"])[None],
                            np.array(c["uniforms"], np.float32)[None])
        assert out[0].tolist() == c["out_ids"], c["name"]
        assert path[0].tolist() == c["path"], c["name"]
        assert n[0] == c["n_accepted"], c["name"]


def test_chain_trees_equal_spec_verify():
    vin = workloads.verify_config("tiny", batch=16)
    p = vin.p.numpy().astype(np.float64)
    q = vin.q.numpy().astype(np.float64)
    ids = vin.draft_ids.numpy()
    u = OS.uniforms_with_margin(p, q, ids, vin.uniforms.numpy(), np.random.default_rng(9))
    B, k1, V = p.shape
    k = k1 - 1
    chain_out, chain_n = vap.spec_verify(_t(p, np.float32), _t(q, np.float32), _t(ids, np.int32), _t(u, np.float32))
    parents = np.tile(np.arange(k + 1) - 1, (B, 1))
    tokens = np.concatenate([np.full((B, 1), -1), ids], axis=1)
    q_tree = np.concatenate([q, np.full((B, 1, V), 1.0 / V)], axis=1)
    u_tree = np.concatenate([u[:, k:], u[:, :k]], axis=1)
    out, path, n = _gpu(p, q_tree, parents, tokens, u_tree)
    assert np.array_equal(n, chain_n.cpu().numpy())
    assert np.array_equal(out, chain_out.cpu().numpy())


def test_scalar_path_and_widest_tree():
    """V not a multiple of 4 (scalar loads) and a 64-node tree."""
    rng = np.random.default_rng(77)
    B, N, V = 6, 64, 3001
    pl = 2.0 * rng.standard_normal((B, N, V))
    ql = pl + 0.8 * rng.standard_normal((B, N, V))
    soft = lambda z: (np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True))
    parents = np.stack([workloads.random_tree_parents(rng, N) for _ in range(B)])
    tin = workloads.make_tree_verify_from_probs(5, soft(pl).astype(np.float32), soft(ql).astype(np.float32), parents)
    _compare(*_margin(tin, 4), "V 3001, 64 nodes")


def test_large_vocabulary():
    """V = 2^20 with 16-node trees."""
    rng = np.random.default_rng(2022)
    B, N, V = 2, 16, 1 << 20
    pl = 3.0 * rng.standard_normal((B, N, V))
    ql = pl + 0.7 * rng.standard_normal((B, N, V))
    soft = lambda z: (np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True))
    parents = np.stack([workloads.random_tree_parents(rng, N) for _ in range(B)])
    tin = workloads.make_tree_verify_from_probs(2022, soft(pl).astype(np.float32), soft(ql).astype(np.float32), parents)
    _compare(*_margin(tin, 13), "V=2^20, 16 nodes")


def test_invalid_parent_sets_error_and_is_ignored():
    tin = workloads.tree_verify_config("tiny_tree", batch=2)
    p, q, parents, tokens, u = _margin(tin, 6)
    bad = parents.copy()
    bad[1, 5] = 7                              # a parent after its child
    ws = vap.tree_verify_workspace(2, DEV)
    out, path, n = vap.spec_verify_tree(_t(p, np.float32), _t(q, np.float32), _t(bad, np.int32),
                                        _t(tokens, np.int32), _t(u, np.float32), workspace=ws)
    assert vap.get_device_error(ws, clear=True) & vap.DERR_TREE
    ref = OT.tree_verify(p[:1], q[:1], parents[:1], tokens[:1], u[:1].astype(np.float64))
    assert np.array_equal(out[:1].cpu().numpy(), ref[0]) and np.array_equal(n[:1].cpu().numpy(), ref[2])


def test_monte_carlo_first_token_follows_the_root_target():
    """4096 copies of one small tree with children drawn from q and raw uniforms: the first
    emitted token is distributed as p(root) (chi-square at the 0.999 quantile)."""
    rng = np.random.default_rng(123)
    V, B = 8, 1 << 12
    parents = np.array([-1, 0, 0, 0, 1, 1, 2])
    N = parents.size
    soft = lambda z: np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    p_nodes = np.stack([soft(1.5 * rng.standard_normal(V)) for _ in range(N)])
    q_nodes = np.stack([soft(1.5 * rng.standard_normal(V)) for _ in range(N)])
    p = np.broadcast_to(p_nodes, (B, N, V)).astype(np.float32)
    q = np.broadcast_to(q_nodes, (B, N, V)).astype(np.float32)
    tokens = np.full((B, N), -1)
    for i in range(1, N):
        w = q_nodes[parents[i]].astype(np.float64)
        tokens[:, i] = rng.choice(V, size=B, p=w / w.sum())
    u = workloads.open_uniforms(rng, (B, N))
    out, path, n = _gpu(p, q, np.broadcast_to(parents, (B, N)), tokens, u)
    counts = np.bincount(out[:, 0], minlength=V)
    exp = B * p_nodes[0].astype(np.float64) / p_nodes[0].sum()
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < stats.chi2.ppf(0.999, V - 1), f"chi2 {chi2}"


def test_one_workspace_across_shapes():
    """One workspace serves five calls of different shapes (vocabularies 300000, 140000, 3001 and
    32768; 8 to 16 nodes): each call leaves the tickets and published slots at zero for the next,
    each is bit-exact, and no device error is set (in particular no VAP_DERR_SYNC)."""
    ws = vap.tree_verify_workspace(64, DEV)
    shapes = [(3, 16, 300000, 31), (32, 8, 140000, 32), (3, 16, 300000, 33), (5, 12, 3001, 34), (16, 16, 32768, 35)]
    for B, N, V, seed in shapes:
        rng = np.random.default_rng(seed)
        pl = 3.0 * rng.standard_normal((B, N, V))
        ql = pl + 0.7 * rng.standard_normal((B, N, V))
        soft = lambda z: np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True)
        parents = np.stack([workloads.random_tree_parents(rng, N) for _ in range(B)])
        tin = workloads.make_tree_verify_from_probs(seed, soft(pl).astype(np.float32), soft(ql).astype(np.float32),
                                                    parents)
        p, q, par, tok, u = _margin(tin, seed)
        ref = OT.tree_verify(p, q, par, tok, u.astype(np.float64))
        got = _gpu(p, q, par, tok, u, workspace=ws)
        for name, a, b in zip(("ids", "path", "n_accepted"), got, ref):
            assert np.array_equal(a, b), f"B={B} N={N} V={V}: {name} differ\n{a}\n{b}"
        assert vap.get_device_error(ws) == 0, f"B={B} N={N} V={V}: device error"


# ---- the draw's fallback branches, bit-exact against the oracle

def _soft(rng, shape, scale=2.0):
    z = scale * rng.standard_normal(shape)
    e = np.exp(z - z.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def _draw_uniform_with_margin(p, q, parents, tokens, u, rng):
    """Keep the accept-test uniforms as given; redraw only u_0 until the walk's every threshold
    is at least 1e-6 away."""
    u = u.copy()
    for b in range(u.shape[0]):
        while OT.tree_decision_margin(p[b], q[b], parents[b], tokens[b], u[b]) < 1e-6:
            u[b, 0] = workloads.open_uniforms(rng, (1,))[0]
    return u


@pytest.mark.parametrize("V", [128256, 3001])
def test_empty_residual_keeps_the_current_distribution(V):
    """The root's target row is half its draft row (used as given), so every residual at the
    root is empty and the walk keeps p_cur = p[root] (the reading for an empty residual).  When
    every child of the root is rejected, the draw kernel finds the weights max(0, p - c' q)
    empty and falls back to the previous c."""
    rng = np.random.default_rng(80 + V)
    B = 16
    parents = np.tile(np.array([-1, 0, 0, 0, 1, 1]), (B, 1))
    N = parents.shape[1]
    q = _soft(rng, (B, N, V))
    p = _soft(rng, (B, N, V))
    p[:, 0] = 0.5 * q[:, 0]                            # exact in fp32
    tokens = np.full((B, N), -1)
    for b in range(B):
        for i in range(1, N):
            w = q[b, parents[b, i]].astype(np.float64)
            tokens[b, i] = rng.choice(V, p=w / w.sum())
    u = workloads.open_uniforms(rng, (B, N))
    u[: B // 2, 1:4] = 0.75                            # the root's three children are rejected
    u[B // 2:, 1] = 0.25                               # child 1 accepted: the walk goes on under it
    u = _draw_uniform_with_margin(p, q, parents, tokens, u, rng)
    ws = vap.tree_verify_workspace(B, DEV)
    ref = OT.tree_verify(p, q, parents, tokens, u.astype(np.float64))
    got = _gpu(p, q, parents, tokens, u, workspace=ws)
    for name, a, b_ in zip(("ids", "path", "n_accepted"), got, ref):
        assert np.array_equal(a, b_), f"V={V}: {name} differ\n{a}\n{b_}"
    assert np.all(ref[2][: B // 2] == 0) and np.all(ref[2][B // 2:] >= 1)
    assert vap.get_device_error(ws) == 0


def test_all_zero_row_emits_token_zero_and_flags():
    """An all-zero target row at the node where the walk ends: the residual and the fallback are
    both empty, so the token is 0 and VAP_DERR_EMPTY_ROW is set.  Sequences 0 and 1 reject every
    child of an all-zero root (P = 0); sequence 2 is an ordinary chain."""
    rng = np.random.default_rng(90)
    V = 128256
    parents = np.array([[-1, 0, 0], [-1, 0, 0], [-1, 0, 1]])
    q = _soft(rng, (3, 3, V))
    p = _soft(rng, (3, 3, V))
    p[0, 0] = 0.0
    p[1, 0] = 0.0
    tokens = np.array([[-1, 5, 9], [-1, 3, 4], [-1, int(np.argmax(q[2, 0])), int(np.argmax(q[2, 1]))]])
    u = workloads.open_uniforms(rng, (3, 3))
    u = _draw_uniform_with_margin(p, q, parents, tokens, u, rng)
    ws = vap.tree_verify_workspace(3, DEV)
    ref = OT.tree_verify(p, q, parents, tokens, u.astype(np.float64))
    got = _gpu(p, q, parents, tokens, u, workspace=ws)
    for name, a, b_ in zip(("ids", "path", "n_accepted"), got, ref):
        assert np.array_equal(a, b_), f"{name} differ\n{a}\n{b_}"
    assert got[0][0, 0] == 0 and got[0][1, 0] == 0 and got[2][0] == 0 and got[2][1] == 0
    assert vap.get_device_error(ws, clear=True) & vap.DERR_EMPTY_ROW
    assert vap.get_device_error(ws) == 0


def test_one_buffer_with_changing_workspace_sizes():
    """Each call passes exactly the bytes its own batch needs, so the size passed changes from
    call to call: bit-exact every time, no device error."""
    lib = vap.load_library()
    shapes = [(24, 8, 140000, 41), (2, 12, 300000, 42), (1, 5, 70000, 43), (32, 8, 140000, 44), (4, 16, 3001, 45),
              (24, 8, 140000, 46)]
    buf = torch.zeros(max(lib.vap_tree_verify_workspace_bytes(s[0]) for s in shapes), dtype=torch.uint8, device=DEV)
    for B, N, V, seed in shapes:
        rng = np.random.default_rng(seed)
        pl = 3.0 * rng.standard_normal((B, N, V))
        ql = pl + 0.7 * rng.standard_normal((B, N, V))
        soft = lambda z: np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True)
        parents = np.stack([workloads.random_tree_parents(rng, N) for _ in range(B)])
        tin = workloads.make_tree_verify_from_probs(seed, soft(pl).astype(np.float32), soft(ql).astype(np.float32),
                                                    parents)
        p, q, par, tok, u = _margin(tin, seed)
        nbytes = lib.vap_tree_verify_workspace_bytes(B)
        print("workspace bytes", nbytes, (B, N, V), flush=True)
        ref = OT.tree_verify(p, q, par, tok, u.astype(np.float64))
        got = _gpu(p, q, par, tok, u, workspace=buf[:nbytes])
        for name, a, b_ in zip(("ids", "path", "n_accepted"), got, ref):
            assert np.array_equal(a, b_), f"B={B} N={N} V={V}: {name} differ\n{a}\n{b_}"
    assert vap.get_device_error(buf) == 0


def test_walk_with_two_chunks_per_workgroup():
    """40 sequences at V = 128256: 16 chunks per residual sum shared by 12 workgroups per
    sequence, so four of them sum two chunks of every shared sum (the two-chunk form) and the
    others one; trees of 5 nodes whose root has four children, so sums are shared."""
    rng = np.random.default_rng(4040)
    B, N, V = 40, 5, 128256
    pl = 3.0 * rng.standard_normal((B, N, V))
    ql = pl + 0.7 * rng.standard_normal((B, N, V))
    soft = lambda z: (np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True))
    parents = np.tile(np.array([-1, 0, 0, 0, 0]), (B, 1))
    tin = workloads.make_tree_verify_from_probs(4040, soft(pl).astype(np.float32), soft(ql).astype(np.float32), parents)
    n = _compare(*_margin(tin, 14), "B=40, V=128256, two chunks per workgroup")
    assert (n == 0).any()   # some roots reject children, so residual sums are taken
