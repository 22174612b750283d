"""Pins of the oracle's verification from logits (CPU only).

* Hand-worked cases (tests/golden/logits_verify_worked.json): temperature 1 and 2, greedy with
  ties.
* The tempered softmax equals scipy.special.softmax(z / T), also for logits of size 1e4 where
  exponentiating without the max shift overflows.
* At T > 0 the result is the probability verifier (oracle.spec_verify, itself pinned) run on
  scipy's softmax of z / T.
* Invariances: a per-row constant added to the logits, and (c z, c T), change nothing.
* T = 0 is exact token matching: drafts accepted exactly while they equal the target row's
  argmax (ties to the smaller id, as numpy.argmax), the emitted token is the argmax of row n;
  a tiny positive T with well-separated logits gives the same result.
* Lossless at T = 0.8: with drafts drawn from softmax(z_q / T), the first emitted token follows
  softmax(z_p / T) (Pearson chi-square at the 0.999 quantile).
"""

import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import chi2

import workloads
from oracle import logits_verify as L
from oracle import spec_verify as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_golden_worked_cases(golden_dir=GOLDEN):
    with open(os.path.join(golden_dir, "logits_verify_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out, n = L.verify_logits_sequence(np.array(c["zp"], np.float32), np.array(c["zq"], np.float32),
                                          c["drafts"], np.array(c["uniforms"], np.float32), c["T"])
        assert out.tolist() == c["out_ids"], c["name"]
        assert n == c["n_accepted"], c["name"]


@pytest.mark.parametrize("T", [1.0, 0.37, 2.5])
def test_tempered_softmax_is_scipy(T):
    rng = np.random.default_rng(3)
    z = (3 * rng.standard_normal((5, 700))).astype(np.float32)
    z[2] += 1e4                      # huge logits: exp without the max shift overflows
    z[3, 17] = -1e4
    ref = sp_softmax(z.astype(np.float64) / T, axis=-1)
    got = L.tempered_softmax(z, T)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("seed", range(4))
def test_positive_temperature_is_the_probability_verifier(seed):
    inp = workloads.logits_verify_config("tiny", seed=500 + seed, batch=6, temps=[1.0, 0.7, 1.3, 0.5, 2.0, 1.0])
    zp, zq, ids = inp.zp.numpy(), inp.zq.numpy(), inp.draft_ids.numpy()
    for b in range(6):
        T = float(inp.temps[b])
        p = sp_softmax(zp[b].astype(np.float64) / T, axis=-1)
        q = sp_softmax(zq[b].astype(np.float64) / T, axis=-1)
        u = S.uniforms_with_margin(p[None], q[None], ids[b][None], inp.uniforms.numpy()[b][None],
                                   np.random.default_rng(seed))[0]
        ref = S.verify_sequence(p, q, ids[b], u)
        got = L.verify_logits_sequence(zp[b], zq[b], ids[b], u, T)
        assert got[1] == ref[1] and got[0].tolist() == ref[0].tolist()


def test_shift_and_scale_invariance():
    inp = workloads.logits_verify_config("tiny", seed=77, batch=8, temps=np.full(8, 0.9))
    zp, zq, ids = inp.zp.numpy().astype(np.float64), inp.zq.numpy().astype(np.float64), inp.draft_ids.numpy()
    u = L.uniforms_with_margin(zp, zq, ids, inp.uniforms.numpy(), inp.temps.numpy(), np.random.default_rng(1))
    base = L.verify_logits(zp, zq, ids, u, inp.temps.numpy())
    rng = np.random.default_rng(2)
    shifted = L.verify_logits(zp + rng.uniform(-50, 50, zp.shape[:2])[..., None],
                              zq + rng.uniform(-50, 50, zq.shape[:2])[..., None], ids, u, inp.temps.numpy())
    scaled = L.verify_logits(4.0 * zp, 4.0 * zq, ids, u, 4.0 * inp.temps.numpy())
    for other in (shifted, scaled):
        assert np.array_equal(other[0], base[0]) and np.array_equal(other[1], base[1])


def _greedy_by_hand(zp, drafts):
    out = []
    for i, x in enumerate(drafts):
        a = int(np.argmax(zp[i]))
        if x != a:
            return out + [a], i
        out.append(int(x))
    return out + [int(np.argmax(zp[len(drafts)]))], len(drafts)


def test_zero_temperature_is_exact_matching():
    rng = np.random.default_rng(9)
    V, k = 12, 4
    for trial in range(200):
        zp = rng.integers(0, 4, (k + 1, V)).astype(np.float32)     # many ties
        zq = rng.standard_normal((k, V)).astype(np.float32)
        # drafts: mostly the target argmax, sometimes another token
        drafts = [int(np.argmax(zp[i])) if rng.random() < 0.7 else int(rng.integers(V)) for i in range(k)]
        u = workloads.open_uniforms(rng, k + 1)
        out, n = L.verify_logits_sequence(zp, zq, drafts, u, 0.0)
        ref, rn = _greedy_by_hand(zp, drafts)
        assert n == rn and out[:n + 1].tolist() == ref and all(out[n + 1:] == -1)


def test_small_temperature_approaches_greedy():
    rng = np.random.default_rng(10)
    V, k = 50, 4
    for trial in range(50):
        zp = rng.permutation(V)[None].repeat(k + 1, 0).astype(np.float32) * 0.1    # gaps of 0.1
        zp = np.stack([rng.permutation(r) for r in zp])
        zq = np.stack([rng.permutation(V) for _ in range(k)]).astype(np.float32) * 0.1
        drafts = [int(np.argmax(zp[i])) if rng.random() < 0.7 else int(np.argmax(zq[i])) for i in range(k)]
        u = workloads.open_uniforms(rng, k + 1)
        greedy = L.verify_logits_sequence(zp, zq, drafts, u, 0.0)
        cold = L.verify_logits_sequence(zp, zq, drafts, u, 1e-4)
        assert cold[1] == greedy[1] and cold[0].tolist() == greedy[0].tolist()


def test_lossless_first_token_at_temperature():
    rng = np.random.default_rng(2024)
    V, k, T, trials = 6, 3, 0.8, 1 << 14
    zp = 1.5 * rng.standard_normal((k + 1, V))
    zq = 1.5 * rng.standard_normal((k, V))
    qd = sp_softmax(zq / T, axis=-1)
    counts = np.zeros(V)
    for _ in range(trials):
        drafts = [int(rng.choice(V, p=qd[i])) for i in range(k)]
        out, n = L.verify_logits_sequence(zp, zq, drafts, rng.random(k + 1), T)
        counts[out[0]] += 1
    exp = trials * sp_softmax(zp[0] / T)
    stat = float(((counts - exp) ** 2 / exp).sum())
    assert stat < chi2.ppf(0.999, V - 1), stat


def test_negative_or_nan_temperature_is_rejected():
    z = np.zeros((2, 3), np.float32)
    for T in (-1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            L.verify_logits_sequence(z, z[:1], [0], [0.5, 0.5], T)
