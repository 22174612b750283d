"""GPU parity of spec_verify against the sequential fp64 oracle (through the C ABI).

Bar: accepted counts and token ids bit-exact, with uniforms placed at least 1e-6 from every
decision threshold the oracle evaluates (oracle.spec_verify.uniforms_with_margin).  A Monte
Carlo test with raw uniforms checks the GPU sampler's emitted distribution directly.
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

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _margin_inputs(vin: workloads.VerifyInputs, seed: int, eps: float = 1e-6):
    p = vin.p.numpy().astype(np.float64)
    q = vin.q.numpy().astype(np.float64)
    ids = vin.draft_ids.numpy()
    u = OS.uniforms_with_margin(p, q, ids, vin.uniforms.numpy(), np.random.default_rng(seed), eps)
    return p, q, ids, u


def _gpu(p32, q32, ids, u, workspace=None):
    p_t = torch.as_tensor(np.ascontiguousarray(p32, dtype=np.float32), device=DEV)
    q_t = torch.as_tensor(np.ascontiguousarray(q32, dtype=np.float32), device=DEV)
    i_t = torch.as_tensor(np.ascontiguousarray(ids, dtype=np.int32), device=DEV)
    u_t = torch.as_tensor(np.ascontiguousarray(u, dtype=np.float32), device=DEV)
    out, n = vap.spec_verify(p_t, q_t, i_t, u_t, workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy(), n.cpu().numpy()


def _compare(p, q, ids, u, what, workspace=None):
    ref_out, ref_n = OS.spec_verify(p, q, ids, u.astype(np.float64))
    out, n = _gpu(p, q, ids, u, workspace)
    assert np.array_equal(n, ref_n), f"{what}: n_accepted {n} vs {ref_n}"
    assert np.array_equal(out, ref_out), f"{what}: ids differ\n{out}\n{ref_out}"
    return ref_n


def test_tiny_config_bit_exact():
    vin = workloads.verify_config("tiny")
    p, q, ids, u = _margin_inputs(vin, 1)
    _compare(p, q, ids, u, "tiny")


def test_spec_verify_step_full_size_bit_exact():
    vin = workloads.verify_config("spec_verify_step")
    p, q, ids, u = _margin_inputs(vin, 2)
    n = _compare(p, q, ids, u, "spec_verify_step")
    print("accepted per sequence", n.tolist(), flush=True)


@pytest.mark.parametrize("seed", range(6))
def test_tiny_recipe_many_seeds(seed):
    vin = workloads.verify_config("tiny", seed=seed, batch=32)
    p, q, ids, u = _margin_inputs(vin, seed)
    _compare(p, q, ids, u, f"tiny seed {seed}")


def test_golden_cases_on_gpu():
    path = os.path.join(os.path.dirname(__file__), "golden", "spec_verify_worked.json")
    for c in json.load(open(path))["cases"]:
        p = np.array(c["p"], dtype=np.float32)[None]
        V = p.shape[2]
        k = len(c["draft_ids"])
        q = np.array(c["q"], dtype=np.float32).reshape(1, k, V)
        ids = np.array(c["draft_ids"], dtype=np.int32).reshape(1, k)
        u = np.array(c["uniforms"], dtype=np.float32)[None]
        if k == 0:
            p_t = torch.as_tensor(p, device=DEV)
            u_t = torch.as_tensor(u, device=DEV)
            out, n = vap.spec_verify(p_t, None, None, u_t)
            out, n = out.cpu().numpy(), n.cpu().numpy()
        else:
            out, n = _gpu(p, q, ids, u)
        assert out[0].tolist() == c["out_ids"], c["name"]
        assert int(n[0]) == c["n_accepted"], c["name"]


def test_p_equal_q_accepts_all_and_zero_prob_rejects():
    rng = np.random.default_rng(3)
    B, k, V = 64, 4, 3001                      # V not a multiple of 4: scalar load path
    logits = 2.0 * rng.standard_normal((B, k + 1, V))
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    q = p[:, :k].copy()
    q64 = q.astype(np.float64)
    ids = np.array([[rng.choice(V, p=q64[b, i] / q64[b, i].sum()) for i in range(k)]
                    for b in range(B)], dtype=np.int32)
    vin = workloads.VerifyInputs("pq", 0, torch.from_numpy(p), torch.from_numpy(q), torch.from_numpy(ids),
                                 torch.from_numpy(workloads.open_uniforms(rng, (B, k + 1))))
    p64, q64, ids, u = _margin_inputs(vin, 4)
    n = _compare(p64, q64, ids, u, "p == q")
    assert np.all(n == k)
    # zero target probability at a draft position -> rejected there
    p2 = p.copy()
    j = rng.integers(0, k, size=B)
    for b in range(B):
        p2[b, j[b], ids[b, j[b]]] = 0.0
    vin2 = workloads.VerifyInputs("zero", 0, torch.from_numpy(p2), torch.from_numpy(q), torch.from_numpy(ids),
                                  torch.from_numpy(u))
    p64, q64, ids2, u2 = _margin_inputs(vin2, 5)
    n2 = _compare(p64, q64, ids2, u2, "p(x) = 0")
    assert np.all(n2 <= j)


def test_greedy_one_hot_rows():
    rng = np.random.default_rng(6)
    B, k, V = 128, 5, 512
    tgt = rng.integers(0, V, size=(B, k + 1))
    ids = np.where(rng.random((B, k)) < 0.7, tgt[:, :k], rng.integers(0, V, size=(B, k))).astype(np.int32)
    p = np.zeros((B, k + 1, V), np.float32)
    q = np.zeros((B, k, V), np.float32)
    for b in range(B):
        p[b, np.arange(k + 1), tgt[b]] = 1.0
        q[b, np.arange(k), ids[b]] = 1.0
    u = workloads.open_uniforms(rng, (B, k + 1))
    out, n = _gpu(p, q, ids, u)
    for b in range(B):
        m = next((i for i in range(k) if ids[b, i] != tgt[b, i]), k)
        assert n[b] == m
        assert out[b, :m].tolist() == ids[b, :m].tolist()
        assert out[b, m] == tgt[b, m]
        assert np.all(out[b, m + 1:] == -1)


def test_k_zero_is_plain_inverse_cdf():
    rng = np.random.default_rng(7)
    B, V = 40, 128256
    logits = 3.0 * rng.standard_normal((B, 1, V))
    p = np.exp(logits - logits.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    vin = workloads.VerifyInputs("k0", 0, torch.from_numpy(p), torch.zeros(B, 0, V),
                                 torch.zeros(B, 0, dtype=torch.int32),
                                 torch.from_numpy(workloads.open_uniforms(rng, (B, 1))))
    p64, q64, ids, u = _margin_inputs(vin, 8)
    p_t = torch.as_tensor(p, device=DEV)
    out, n = vap.spec_verify(p_t, None, None, torch.as_tensor(u, device=DEV))
    ref_out, ref_n = OS.spec_verify(p64, q64, ids, u.astype(np.float64))
    assert np.array_equal(out.cpu().numpy(), ref_out) and np.all(n.cpu().numpy() == 0)


def test_out_of_range_draft_sets_error_and_rejects():
    vin = workloads.verify_config("tiny")
    p, q, ids, u = _margin_inputs(vin, 9)
    ids = ids.copy()
    ids[2, 0] = 5000
    ids[3, 1] = -3
    ws = vap.verify_workspace(4, 4, 1000, DEV)
    ref_n = _compare(p, q, ids, u, "bad ids", workspace=ws)
    assert ref_n[2] == 0 and ref_n[3] <= 1
    assert vap.get_device_error(ws, clear=True) & vap.DERR_DRAFT_ID
    assert vap.get_device_error(ws) == 0


def test_workspace_reuse_and_batch_sweep():
    """Same workspace, several batch sizes in a row (arrival counters must reset)."""
    ws = vap.verify_workspace(256, 4, 32000, DEV)
    for B in (1, 7, 256, 16):
        rng = np.random.default_rng(B)
        pl = 3.0 * rng.standard_normal((B, 5, 32000))
        ql = pl[:, :4] + 0.7 * rng.standard_normal((B, 4, 32000))
        vin = workloads.make_verify_inputs(B, p_logits=pl, q_logits=ql, rng=rng)
        p, q, ids, u = _margin_inputs(vin, B)
        _compare(p, q, ids, u, f"B={B}", workspace=ws)


def test_large_batch_small_vocab():
    """B = 4096 sequences of a 1000-token vocabulary: one chunk per row, one workgroup each."""
    vin = workloads.verify_config("tiny", seed=77, batch=4096)
    p, q, ids, u = _margin_inputs(vin, 5)
    _compare(p, q, ids, u, "B=4096")


def test_batch_with_thirty_two_chunks_per_workgroup():
    """256 sequences at V = 128256: 126 chunks of 1020 tokens per row, four workgroups per
    sequence, so each workgroup streams 32 consecutive chunks (eight per wave) -- the count from
    which the chunk loads take the non-temporal path."""
    vin = workloads.verify_config("spec_verify_step", seed=4242, batch=256)
    p, q, ids, u = _margin_inputs(vin, 4243)
    _compare(p, q, ids, u, "B=256, V=128256")


def test_largest_vocabulary():
    """V = 2^20, the largest vocabulary: 256 chunks of 4096 tokens per row."""
    rng = np.random.default_rng(2020)
    B, k, V = 2, 4, 1 << 20
    pl = 3.0 * rng.standard_normal((B, k + 1, V))
    ql = pl[:, :k] + 0.7 * rng.standard_normal((B, k, V))
    vin = workloads.make_verify_inputs(2020, p_logits=pl, q_logits=ql, rng=rng)
    p, q, ids, u = _margin_inputs(vin, 11)
    _compare(p, q, ids, u, "V=2^20")


def test_vocabulary_with_chunks_of_two_pieces_not_a_multiple_of_four():
    """V = 300001: 256 chunks of 1172 tokens, each summed by one wave in two pieces (1024 + 148),
    with the scalar (not 16-byte) loads, and the select over 16 tokens per thread."""
    rng = np.random.default_rng(3001)
    B, k, V = 3, 4, 300001
    pl = 3.0 * rng.standard_normal((B, k + 1, V))
    ql = pl[:, :k] + 0.7 * rng.standard_normal((B, k, V))
    vin = workloads.make_verify_inputs(3001, p_logits=pl, q_logits=ql, rng=rng)
    p, q, ids, u = _margin_inputs(vin, 12)
    _compare(p, q, ids, u, "V=300001")


def test_monte_carlo_emitted_distribution():
    """Raw uniforms, 2^18 sequences sharing fixed p_j, q_j (V = 8, k = 4): the tokens the GPU
    emits at each position follow p_j (chi-square at the 0.999 quantile)."""
    rng = np.random.default_rng(11)
    N, k, V = 1 << 18, 4, 8
    pl = 2.0 * rng.standard_normal((k + 1, V))
    ql = 2.0 * rng.standard_normal((k, V))
    p = np.exp(pl - pl.max(-1, keepdims=True)); p /= p.sum(-1, keepdims=True)
    q = np.exp(ql - ql.max(-1, keepdims=True)); q /= q.sum(-1, keepdims=True)
    p32, q32 = p.astype(np.float32), q.astype(np.float32)
    ids = np.stack([rng.choice(V, size=N, p=q32[i].astype(np.float64) / q32[i].sum()) for i in range(k)], 1)
    u = workloads.open_uniforms(rng, (N, k + 1))
    P = np.broadcast_to(p32, (N, k + 1, V))
    Qm = np.broadcast_to(q32, (N, k, V))
    out, n = _gpu(P, Qm, ids.astype(np.int32), u)
    crit = stats.chi2.ppf(0.999, V - 1)
    pn = p32.astype(np.float64)
    for j in range(k + 1):
        reached = n >= j
        counts = np.bincount(out[reached, j], minlength=V)
        expected = counts.sum() * pn[j] / pn[j].sum()
        chi2 = float(((counts - expected) ** 2 / expected).sum())
        assert chi2 < crit, (j, chi2)
    alpha = np.minimum(p32[:k], q32).astype(np.float64).sum(1)
    for i in range(k):
        reached = n >= i
        rate = (n[reached] > i).mean()
        sd = np.sqrt(alpha[i] * (1 - alpha[i]) / reached.sum())
        assert abs(rate - alpha[i]) < 5 * sd


# ---- the draw's fallback branches (the oracle's readings for an empty residual, an all-zero
# ---- row and a threshold at or past the total), each bit-exact against the oracle

def _softmax_rows(rng, shape, scale=2.0):
    z = scale * rng.standard_normal(shape)
    e = np.exp(z - z.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("V", [128256, 3001])
def test_empty_residual_falls_back_to_the_target_row(V):
    """p_i = q_i / 2 (used as given) makes every residual max(0, p - q) empty: a rejection at n
    draws from p_n itself, the last workgroup recomputing its chunk sums; V = 3001 runs the
    scalar load path."""
    rng = np.random.default_rng(40 + V)
    B, k = 24, 4
    q = _softmax_rows(rng, (B, k, V))
    p = np.empty((B, k + 1, V), np.float32)
    p[:, :k] = 0.5 * q                                # exact in fp32
    p[:, k] = _softmax_rows(rng, (B, V))
    ids = np.array([[rng.choice(V, p=q[b, i].astype(np.float64) / q[b, i].astype(np.float64).sum())
                     for i in range(k)] for b in range(B)], dtype=np.int32)
    u0 = workloads.open_uniforms(rng, (B, k + 1))
    u = OS.uniforms_with_margin(p.astype(np.float64), q.astype(np.float64), ids, u0, rng)
    ws = vap.verify_workspace(B, k, V, DEV)
    n = _compare(p.astype(np.float64), q.astype(np.float64), ids, u, f"empty residual V={V}", workspace=ws)
    assert np.any(n < k), "no sequence took the fallback"
    assert vap.get_device_error(ws) == 0
    print("accepted", n.tolist(), flush=True)


@pytest.mark.parametrize("V", [128256, 1000])
def test_all_zero_row_emits_token_zero_and_flags(V):
    """A rejection on an all-zero target row (residual and fallback both empty), and a bonus
    draw from an all-zero row: token 0 and VAP_DERR_EMPTY_ROW; the other sequences are
    unaffected."""
    rng = np.random.default_rng(50 + V)
    B, k = 6, 3
    q = _softmax_rows(rng, (B, k, V))
    p = _softmax_rows(rng, (B, k + 1, V))
    ids = np.argmax(q, axis=-1).astype(np.int32)
    p[1, 0] = 0.0                                     # draft 0 of sequence 1: P = 0, rejected
    p[3, :k] = q[3]                                   # sequence 3 accepts every draft ...
    p[3, k] = 0.0                                     # ... and its bonus row is empty
    u0 = workloads.open_uniforms(rng, (B, k + 1))
    keep = np.ones(B, bool)
    keep[[1, 3]] = False
    u = u0.copy()
    u[keep] = OS.uniforms_with_margin(p[keep].astype(np.float64), q[keep].astype(np.float64), ids[keep],
                                      u0[keep], rng)
    ws = vap.verify_workspace(B, k, V, DEV)
    n = _compare(p.astype(np.float64), q.astype(np.float64), ids, u, f"all-zero rows V={V}", workspace=ws)
    assert n[1] == 0 and n[3] == k
    out, _ = _gpu(p, q, ids, u, ws)
    assert out[1, 0] == 0 and out[3, k] == 0
    assert vap.get_device_error(ws, clear=True) & vap.DERR_EMPTY_ROW
    assert vap.get_device_error(ws) == 0


def test_threshold_past_the_total_takes_the_last_positive_token():
    """An infinite weight makes t = u * Z infinite, so no running sum exceeds it: both sides
    take the largest token with positive weight (the reading for t at or past the total).  The
    drafts are accepted (p = q), so the bonus row is drawn from."""
    rng = np.random.default_rng(60)
    B, k, V = 5, 2, 128256
    q = _softmax_rows(rng, (B, k, V))
    p = np.empty((B, k + 1, V), np.float32)
    p[:, :k] = q
    p[:, k] = _softmax_rows(rng, (B, V))
    last = [V - 1, 70000, 4095, 4096, 128000]
    for b in range(B):
        p[b, k, 1000 + 37 * b] = np.inf
        p[b, k, last[b] + 1:] = 0.0                   # the last positive token of the row
    ids = np.argmax(q, axis=-1).astype(np.int32)
    u = workloads.open_uniforms(rng, (B, k + 1))
    ref_out, ref_n = OS.spec_verify(p.astype(np.float64), q.astype(np.float64), ids, u.astype(np.float64))
    assert np.all(ref_n == k) and ref_out[:, k].tolist() == last
    out, n = _gpu(p, q, ids, u)
    assert np.array_equal(n, ref_n) and np.array_equal(out, ref_out), (out[:, k], last)


def test_one_buffer_with_changing_workspace_sizes():
    """One buffer, each call passing exactly the bytes its own batch needs (so the size passed
    changes from call to call, and a large call's chunk sums lie where a small call's workspace
    ends): bit-exact every time, no device error."""
    big = vap.load_library().vap_verify_workspace_bytes(256, 4, 128256)
    buf = torch.zeros(big, dtype=torch.uint8, device=DEV)
    lib = vap.load_library()
    for B, V, seed in [(64, 128256, 1), (4, 128256, 2), (1, 32000, 3), (256, 128256, 4), (16, 128256, 5),
                       (4, 5003, 6), (64, 128256, 7)]:
        rng = np.random.default_rng(seed)
        pl = 3.0 * rng.standard_normal((B, 5, V))
        ql = pl[:, :4] + 0.7 * rng.standard_normal((B, 4, V))
        vin = workloads.make_verify_inputs(seed, p_logits=pl, q_logits=ql, rng=rng)
        p, q, ids, u = _margin_inputs(vin, seed)
        nbytes = lib.vap_verify_workspace_bytes(B, 4, V)
        print("workspace bytes", nbytes, "B", B, "V", V, flush=True)
        _compare(p, q, ids, u, f"B={B} V={V} bytes={nbytes}", workspace=buf[:nbytes])
    assert vap.get_device_error(buf) == 0
