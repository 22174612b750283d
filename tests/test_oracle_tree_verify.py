"""Pins of the oracle's tree verification (CPU only).

* Hand-worked cases (tests/golden/tree_verify_worked.json).
* A chain-shaped tree is the chain verifier (oracle.spec_verify, itself pinned), decision for
  decision.
* A root-only tree is a plain inverse-CDF draw (numpy searchsorted).
* Lossless: with each node's children drawn independently from that node's draft row and a
  target that depends only on the token path, the first emitted token follows p(root) and the
  second, given the first, follows the target after it (Pearson chi-square at the 0.999
  quantile).
"""

import json
import os

import numpy as np
import pytest

import workloads
from oracle import spec_verify as S
from oracle import tree_verify as T

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_golden_worked_cases(golden_dir=GOLDEN):
    with open(os.path.join(golden_dir, "tree_verify_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ids, path, n = T.tree_verify_sequence(np.array(c["p"], np.float32), np.array(c["q"], np.float32),
                                              c["parents"], c["tokens"], np.array(c["uniforms"], np.float32))
        assert ids.tolist() == c["out_ids"], c["name"]
        assert path.tolist() == c["path"], c["name"]
        assert n == c["n_accepted"], c["name"]


@pytest.mark.parametrize("seed", range(12))
def test_chain_tree_is_the_chain_verifier(seed):
    rng = np.random.default_rng(seed)
    k, V = int(rng.integers(1, 7)), int(rng.integers(3, 40))
    p = rng.dirichlet(np.full(V, 0.5), size=k + 1).astype(np.float32)
    q = rng.dirichlet(np.full(V, 0.5), size=k).astype(np.float32)
    q64 = q.astype(np.float64)
    drafts = np.array([rng.choice(V, p=q64[i] / q64[i].sum()) for i in range(k)])
    u = workloads.open_uniforms(rng, k + 1)
    ids, n = S.verify_sequence(p, q, drafts, u)
    # tree: node 0 root, node i the draft at position i-1; q row of node u drew node u+1
    parents = np.arange(k + 1) - 1
    tokens = np.concatenate([[-1], drafts])
    q_tree = np.concatenate([q, np.full((1, V), 1.0 / V, np.float32)])
    u_tree = np.concatenate([[u[k]], u[:k]]).astype(np.float32)
    t_ids, path, t_n = T.tree_verify_sequence(p, q_tree, parents, tokens, u_tree)
    assert t_n == n
    assert t_ids[:n + 1].tolist() == ids[:n + 1].tolist()
    assert path[:n].tolist() == list(range(1, n + 1))


@pytest.mark.parametrize("seed", range(5))
def test_root_only_is_numpy_inverse_cdf(seed):
    rng = np.random.default_rng(50 + seed)
    V = 100
    p = rng.dirichlet(np.ones(V)).astype(np.float32)[None]
    u = workloads.open_uniforms(rng, 1)
    ids, path, n = T.tree_verify_sequence(p, p, [-1], [-1], u)
    w = p[0].astype(np.float64)
    expect = int(np.searchsorted(np.cumsum(w), float(u[0]) * w.sum(), side="right"))
    assert n == 0 and ids[0] == expect


def _chi2_ok(counts, probs):
    from scipy.stats import chi2
    n = counts.sum()
    exp = n * probs
    keep = exp > 0
    stat = float((((counts - exp) ** 2)[keep] / exp[keep]).sum())
    df = int(keep.sum()) - 1
    return stat < chi2.ppf(0.999, df), stat


def test_lossless_monte_carlo_on_a_two_level_tree():
    rng = np.random.default_rng(2024)
    V = 5
    soft = lambda z: np.exp(z - z.max(-1, keepdims=True)) / np.exp(z - z.max(-1, keepdims=True)).sum(-1, keepdims=True)
    p_root = soft(1.5 * rng.standard_normal(V))
    q_root = soft(1.5 * rng.standard_normal(V))
    P1 = soft(1.5 * rng.standard_normal((V, V)))       # target after token x
    Q1 = soft(1.5 * rng.standard_normal((V, V)))       # draft after token x
    P2 = soft(1.5 * rng.standard_normal((V, V, V)))    # target after tokens x1 x2
    parents = [-1, 0, 0, 0, 1, 1, 2, 2, 3, 3]          # root, 3 children, 2 grandchildren each
    N = len(parents)
    trials = 1 << 15
    c1 = np.zeros(V)
    c2 = np.zeros((V, V))
    for _ in range(trials):
        tok = np.full(N, -1)
        for i in range(1, N):
            dist = q_root if parents[i] == 0 else Q1[tok[parents[i]]]
            tok[i] = rng.choice(V, p=dist)
        p_rows = np.empty((N, V))
        q_rows = np.empty((N, V))
        for i in range(N):
            if i == 0:
                p_rows[i], q_rows[i] = p_root, q_root
            elif parents[i] == 0:
                p_rows[i], q_rows[i] = P1[tok[i]], Q1[tok[i]]
            else:
                p_rows[i], q_rows[i] = P2[tok[parents[i]], tok[i]], q_root
        ids, path, n = T.tree_verify_sequence(p_rows, q_rows, parents, tok, rng.random(N))
        c1[ids[0]] += 1
        if n >= 1:
            c2[ids[0], ids[1]] += 1
    ok, stat = _chi2_ok(c1, p_root)
    assert ok, f"first token chi2 {stat}"
    for x in range(V):
        if c2[x].sum() > 500:
            ok, stat = _chi2_ok(c2[x], P1[x])
            assert ok, f"second token after {x}: chi2 {stat}"
