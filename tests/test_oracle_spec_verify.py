"""Pins for the speculative-verification oracle (CPU only).

The oracle is checked against hand-worked cases (tests/golden), the invariants the pages fix
(p == q accepts every draft; a draft with zero target probability is rejected; temperature 0
reduces to exact token matching), numpy's inverse-CDF routine for k = 0, the closed-form
acceptance probability sum_x min(p(x), q(x)), an exact stratified enumeration of the emitted
distribution, and a Monte Carlo chi-square test of the lossless-distribution claim.
"""

import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import spec_verify as S


def _softmax(x):
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _probs(rng, shape, sigma=2.0):
    return _softmax(sigma * rng.standard_normal(shape)).astype(np.float32).astype(np.float64)


def test_golden_worked_cases(golden_dir):
    with open(os.path.join(golden_dir, "spec_verify_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p = np.array(c["p"], dtype=np.float32).astype(np.float64)
        V = p.shape[1]
        q = np.array(c["q"], dtype=np.float32).astype(np.float64).reshape(len(c["draft_ids"]), V)
        u = np.array(c["uniforms"], dtype=np.float32)
        out, n = S.verify_sequence(p, q, c["draft_ids"], u)
        assert out.tolist() == c["out_ids"], c["name"]
        assert n == c["n_accepted"], c["name"]


def test_p_equal_q_accepts_every_draft():
    rng = np.random.default_rng(0)
    V, k = 50, 6
    for trial in range(200):
        p = _probs(rng, (k + 1, V))
        q = p[:k].copy()
        drafts = rng.integers(0, V, size=k)
        drafts = np.where(p[np.arange(k), drafts] > 0, drafts, np.argmax(p[:k], axis=1))
        u = rng.random(k + 1)
        u = np.where(u == 0, 0.5, u)
        out, n = S.verify_sequence(p, q, drafts, u)
        assert n == k
        assert out[:k].tolist() == drafts.tolist()
        cum = np.cumsum(p[k])
        assert out[k] == int(np.searchsorted(cum, u[k] * cum[-1], side="right"))


def test_zero_target_probability_is_always_rejected():
    rng = np.random.default_rng(1)
    V, k = 30, 4
    for trial in range(200):
        p = _probs(rng, (k + 1, V))
        q = p[:k].copy()
        j = int(rng.integers(0, k))
        drafts = rng.integers(0, V, size=k)
        x = int(drafts[j])
        p[j, x] = 0.0                               # target gives the draft zero probability
        q[j, x] = max(q[j, x], 1e-3)
        u = rng.random(k + 1) * 0.999 + 0.0005
        out, n = S.verify_sequence(p, q, drafts, u)
        assert n <= j
        if n == j:
            assert out[j] != x                      # residual has zero weight at x


def test_temperature_zero_reduces_to_exact_matching():
    rng = np.random.default_rng(2)
    V, k = 20, 5
    for trial in range(300):
        tgt = rng.integers(0, V, size=k + 1)
        drafts = np.where(rng.random(k) < 0.6, tgt[:k], rng.integers(0, V, size=k))
        p = np.zeros((k + 1, V))
        p[np.arange(k + 1), tgt] = 1.0
        q = np.zeros((k, V))
        q[np.arange(k), drafts] = 1.0
        u = rng.random(k + 1) * 0.998 + 0.001
        out, n = S.verify_sequence(p, q, drafts, u)
        expect_n = k
        for i in range(k):
            if drafts[i] != tgt[i]:
                expect_n = i
                break
        assert n == expect_n
        assert out[:n].tolist() == drafts[:n].tolist()
        assert out[n] == tgt[n]
        assert all(x == -1 for x in out[n + 1:])


def test_k_zero_is_numpy_inverse_cdf():
    rng = np.random.default_rng(3)
    for V in (1, 2, 7, 1000):
        for trial in range(50):
            p = _probs(rng, (1, V))
            u = np.float32(rng.random() * 0.999 + 0.0005)
            out, n = S.verify_sequence(p, np.zeros((0, V)), [], [u])
            cum = np.cumsum(p[0])
            assert n == 0
            assert out[0] == int(np.searchsorted(cum, np.float64(u) * cum[-1], side="right"))


def test_out_of_range_draft_is_rejected():
    p = np.array([[0.3, 0.7], [0.5, 0.5]])
    q = np.array([[0.5, 0.5]])
    for x in (-1, 2, 1 << 30):
        out, n = S.verify_sequence(p, q, [x], [0.01, 0.9])
        assert n == 0 and out.tolist() == [1, -1]


def test_residual_fallback_when_residual_is_empty():
    # p <= q everywhere (not normalised): residual sums to 0 -> the oracle draws from p_n
    p = np.array([[0.1, 0.2, 0.1], [0.3, 0.3, 0.4]])
    q = np.array([[0.5, 0.3, 0.2]])
    out, n = S.verify_sequence(p, q, [0], [0.9, 0.6])   # ratio 0.2 < 0.9 -> reject
    assert n == 0
    cum = np.cumsum(p[0])
    assert out[0] == int(np.searchsorted(cum, np.float64(np.float32(0.6)) * cum[-1], side="right"))


def test_emitted_distribution_exact_by_stratified_enumeration():
    """Brute force over a fine grid of uniforms: P(emit y) == p(y) for one position.

    For every draft token x (weight q(x)) the accept test and the residual draw are evaluated
    on M stratified uniforms, so each frequency is exact to within 1/M.
    """
    rng = np.random.default_rng(4)
    M = 2048
    grid = (np.arange(M) + 0.5) / M
    for V in (3, 5, 8):
        p = _probs(rng, (2, V), sigma=1.5)
        q = _probs(rng, (1, V), sigma=1.5)
        emit = np.zeros(V)
        for x in range(V):
            acc = np.array([S.accept_draft(p[0, x], q[0, x], r) for r in grid]).mean()
            res = np.zeros(V)
            w = np.maximum(0.0, p[0] - q[0])
            for u in grid:
                res[S.sample_inverse_cdf(w, u)] += 1.0 / M
            emit[x] += q[0, x] * acc
            emit += q[0, x] * (1 - acc) * res
        np.testing.assert_allclose(emit, p[0], atol=3.0 / M)


def _monte_carlo(rng, p, q, N):
    k, V = q.shape
    emitted = np.full((N, k + 1), -1)
    nacc = np.empty(N, dtype=np.int64)
    cq = [np.cumsum(q[i]) for i in range(k)]
    for t in range(N):
        drafts = [min(int(np.searchsorted(cq[i], rng.random() * cq[i][-1], side="right")), V - 1)
                  for i in range(k)]
        u = rng.random(k + 1)
        u = np.where(u == 0, 0.5, u)
        out, n = S.verify_sequence(p, q, drafts, u)
        emitted[t] = out
        nacc[t] = n
    return emitted, nacc


@pytest.mark.parametrize("V,N", [(8, 60000), (16, 60000)])
def test_lossless_chi_square_and_acceptance_rate(V, N):
    """Tokens emitted at each position follow p (Pearson chi-square at the 0.999 quantile), and
    the per-position acceptance rate matches sum_x min(p(x), q(x)) within 5 sigma."""
    rng = np.random.default_rng(100 + V)
    k = 4
    p = _probs(rng, (k + 1, V))
    q = _probs(rng, (k, V))
    emitted, nacc = _monte_carlo(rng, p, q, N)
    crit = stats.chi2.ppf(0.999, V - 1)
    for j in range(k + 1):
        reached = nacc >= j
        counts = np.bincount(emitted[reached, j], minlength=V)
        n_j = counts.sum()
        expected = n_j * p[j] / p[j].sum()
        chi2 = float(((counts - expected) ** 2 / expected).sum())
        assert chi2 < crit, (j, chi2, crit)
    alpha = np.minimum(p[:k], q).sum(axis=1)
    for i in range(k):
        reached = nacc >= i
        trials = int(reached.sum())
        accepted = int((nacc[reached] > i).sum())
        sigma = np.sqrt(alpha[i] * (1 - alpha[i]) / trials)
        assert abs(accepted / trials - alpha[i]) < 5 * sigma, (i, accepted / trials, alpha[i])
    # expected emitted count E[n + 1] = sum_j prod_{i<j} alpha_i
    expect_len = sum(np.prod(alpha[:j]) for j in range(k + 1))
    sd = np.sqrt(np.var(nacc + 1) / N)
    assert abs(np.mean(nacc + 1) - expect_len) < 5 * sd


def test_margin_helper_keeps_decisions_stable():
    rng = np.random.default_rng(5)
    B, k, V = 6, 4, 200
    p = np.stack([_probs(rng, (k + 1, V)) for _ in range(B)])
    q = np.stack([_probs(rng, (k, V)) for _ in range(B)])
    drafts = np.array([[int(np.argmax(q[b, i])) for i in range(k)] for b in range(B)])
    u0 = rng.random((B, k + 1)).astype(np.float32)
    u = S.uniforms_with_margin(p, q, drafts, u0, rng, eps=1e-4)
    for b in range(B):
        assert S.decision_margin(p[b], q[b], drafts[b], u[b]) >= 1e-4
        base = S.verify_sequence(p[b], q[b], drafts[b], u[b])
        for delta in (-5e-5, 5e-5):
            moved = S.verify_sequence(p[b], q[b], drafts[b], u[b].astype(np.float64) + delta)
            assert moved[0].tolist() == base[0].tolist() and moved[1] == base[1]
