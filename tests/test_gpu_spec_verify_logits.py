"""GPU parity of spec_verify_logits against the fp64 oracle (through the C ABI).

Bar: emitted ids and accepted counts bit-exact, with uniforms placed at least 1e-6 from every
threshold the oracle evaluates (oracle.logits_verify.uniforms_with_margin).  The kernel takes
its exponentials in fp64 (relative error near 1e-15), far inside that margin.  A Monte Carlo
test with raw uniforms checks the emitted distribution directly.
"""

import json
import os

import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax as sp_softmax

import verify_attention_paged_amd as vap
import workloads
from oracle import logits_verify as OL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _t(x, dt):
    return torch.as_tensor(np.ascontiguousarray(x, dtype=dt), device=DEV)


def _gpu(zp, zq, ids, u, temps, workspace=None):
    k = zp.shape[1] - 1
    out, n = vap.spec_verify_logits(_t(zp, np.float32), _t(zq, np.float32) if k else None,
                                    _t(ids, np.int32) if k else None, _t(u, np.float32), _t(temps, np.float32),
                                    workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy(), n.cpu().numpy()


def _compare(zp, zq, ids, u, temps, what, workspace=None):
    ref = OL.verify_logits(zp, zq, ids, u, temps)
    got = _gpu(zp, zq, ids, u, temps, workspace)
    assert np.array_equal(got[1], ref[1]), f"{what}: n_accepted {got[1]} vs {ref[1]}"
    assert np.array_equal(got[0], ref[0]), f"{what}: ids\n{got[0]}\n{ref[0]}"
    return ref


def _margin(inp, seed):
    zp, zq, ids, T = inp.zp.numpy(), inp.zq.numpy(), inp.draft_ids.numpy(), inp.temps.numpy()
    u = OL.uniforms_with_margin(zp, zq, ids, inp.uniforms.numpy(), T, np.random.default_rng(seed))
    return zp, zq, ids, u, T


def test_tiny_mixed_temperatures_bit_exact():
    _compare(*_margin(workloads.logits_verify_config("tiny"), 1), "tiny")


@pytest.mark.parametrize("seed", range(4))
def test_tiny_many_seeds_and_temperatures(seed):
    rng = np.random.default_rng(seed)
    temps = rng.choice([0.0, 0.3, 0.7, 1.0, 1.6, 3.0], size=24)
    inp = workloads.logits_verify_config("tiny", seed=4000 + seed, batch=24, temps=temps)
    _compare(*_margin(inp, seed), f"tiny seed {seed}")


def test_full_vocab_temperature_one_bit_exact():
    ref = _compare(*_margin(workloads.logits_verify_config("spec_verify_step"), 2), "spec_verify_step")
    print("accepted per sequence", ref[1].tolist(), flush=True)


def test_full_vocab_mixed_temperatures():
    temps = np.array([0.0, 0.5, 1.0, 1.7] * 4)
    inp = workloads.logits_verify_config("spec_verify_step", seed=77, temps=temps)
    _compare(*_margin(inp, 3), "spec_verify_step, mixed temperatures")


def test_golden_cases_on_gpu():
    with open(os.path.join(GOLDEN, "logits_verify_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out, n = _gpu(np.array(c["zp"], np.float32)[None], np.array(c["zq"], np.float32)[None],
                      np.array(c["drafts"])[None], np.array(c["uniforms"], np.float32)[None],
                      np.array([c["T"]], np.float32))
        assert out[0].tolist() == c["out_ids"], c["name"]
        assert n[0] == c["n_accepted"], c["name"]


@pytest.mark.parametrize("V,k", [(3001, 4), (1, 2), (2, 1), (4097, 0), (5000, 8), (8192, 16)])
def test_shapes_scalar_path_and_k(V, k):
    rng = np.random.default_rng(V + k)
    B = 5
    zp = (2.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    zq = (zp[:, :k] + 0.5 * rng.standard_normal((B, k, V))).astype(np.float32)
    temps = np.array([1.0, 0.6, 0.0, 2.0, 1.0])
    inp = workloads.make_logits_verify_inputs(V * 7 + k, zp, zq, temps)
    _compare(*_margin(inp, 5), f"V {V} k {k}")


def test_large_and_masked_logits():
    rng = np.random.default_rng(12)
    B, k, V = 6, 4, 2048
    zp = (3.0 * rng.standard_normal((B, k + 1, V)) + 1e4).astype(np.float32)
    zq = (zp[:, :k] - 2e4 + rng.standard_normal((B, k, V))).astype(np.float32)
    zp[:, :, ::7] = -np.inf                         # masked tokens
    zq[:, :, 3::11] = -np.inf
    temps = np.array([1.0, 0.5, 0.0, 1.3, 1.0, 0.9])
    inp = workloads.make_logits_verify_inputs(99, zp, zq, temps)
    _compare(*_margin(inp, 6), "large / masked logits")


def test_invalid_temperature_is_greedy_and_flagged():
    inp = workloads.logits_verify_config("tiny", seed=8, batch=4, temps=[1.0, 0.0, 1.0, 1.0])
    zp, zq, ids, u, T = _margin(inp, 7)
    bad = T.copy()
    bad[2], bad[3] = -1.0, np.nan
    ws = vap.verify_logits_workspace(4, inp.k, inp.vocab, DEV)
    out, n = _gpu(zp, zq, ids, u, bad, workspace=ws)
    assert vap.get_device_error(ws, clear=True) & vap.DERR_TEMP
    greedy = T.copy()
    greedy[2] = greedy[3] = 0.0
    ref = OL.verify_logits(zp, zq, ids, u, greedy)
    assert np.array_equal(out, ref[0]) and np.array_equal(n, ref[1])


def test_matches_the_probability_path():
    """T = 1 from logits and spec_verify on the oracle's fp64 softmax stored as fp32."""
    inp = workloads.logits_verify_config("tiny", seed=31, batch=32, temps=np.ones(32))
    zp, zq, ids, u, T = _margin(inp, 8)
    p = sp_softmax(zp.astype(np.float64), axis=-1).astype(np.float32)
    q = sp_softmax(zq.astype(np.float64), axis=-1).astype(np.float32)
    out_l, n_l = _gpu(zp, zq, ids, u, T)
    out_p, n_p = vap.spec_verify(_t(p, np.float32), _t(q, np.float32), _t(ids, np.int32), _t(u, np.float32))
    assert np.array_equal(n_l, n_p.cpu().numpy()) and np.array_equal(out_l, out_p.cpu().numpy())


def test_workspace_reuse_across_shapes():
    shapes = [(16, 4, 128256), (1, 0, 7), (64, 2, 1000), (3, 12, 4099), (16, 4, 128256)]
    size = max(vap.load_library().vap_verify_logits_workspace_bytes(B, k, V) for B, k, V in shapes)
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    for i, (B, k, V) in enumerate(shapes):
        rng = np.random.default_rng(100 + i)
        zp = (2.5 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
        zq = (zp[:, :k] + 0.6 * rng.standard_normal((B, k, V))).astype(np.float32)
        temps = rng.choice([0.0, 0.8, 1.0], size=B)
        inp = workloads.make_logits_verify_inputs(200 + i, zp, zq, temps)
        _compare(*_margin(inp, 9 + i), f"call {i} {(B, k, V)}", workspace=ws)


def test_largest_vocabulary():
    """V = 2^20: 512 statistics chunks per row, merged in three LDS passes per sequence."""
    rng = np.random.default_rng(2021)
    B, k, V = 2, 4, 1 << 20
    zp = (3.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    zq = (zp[:, :k] + 0.7 * rng.standard_normal((B, k, V))).astype(np.float32)
    inp = workloads.make_logits_verify_inputs(2021, zp, zq, [1.0, 0.8])
    _compare(*_margin(inp, 12), "V=2^20")


def test_monte_carlo_first_token_at_temperature():
    """4096 copies of one sequence with drafts drawn from softmax(z_q / T) and raw uniforms:
    the first emitted token follows softmax(z_p / T) (chi-square at the 0.999 quantile)."""
    rng = np.random.default_rng(123)
    V, k, B, T = 8, 3, 1 << 12, 0.8
    zp1 = (1.5 * rng.standard_normal((k + 1, V))).astype(np.float32)
    zq1 = (1.5 * rng.standard_normal((k, V))).astype(np.float32)
    qd = sp_softmax(zq1.astype(np.float64) / T, axis=-1)
    ids = np.stack([np.array([rng.choice(V, p=qd[i]) for i in range(k)]) for _ in range(B)])
    u = workloads.open_uniforms(rng, (B, k + 1))
    out, n = _gpu(np.broadcast_to(zp1, (B, k + 1, V)), np.broadcast_to(zq1, (B, k, V)), ids, u, np.full(B, T))
    counts = np.bincount(out[:, 0], minlength=V)
    exp = B * sp_softmax(zp1[0].astype(np.float64) / T)
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < stats.chi2.ppf(0.999, V - 1), f"chi2 {chi2}"


@pytest.mark.parametrize("V", [128256, 3001])
def test_empty_residual_falls_back_to_the_target_row(V):
    """Draft rows equal to the target rows give p = q bit for bit on both sides, so the residual
    after a rejection is empty; an out-of-range draft id forces that rejection.  The token is
    then drawn from p_n (the fallback reading), bit-exact, and VAP_DERR_DRAFT_ID is set."""
    rng = np.random.default_rng(70 + V)
    B, k = 12, 4
    zp = (2.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    zq = zp[:, :k].copy()
    temps = np.where(np.arange(B) % 3 == 0, 0.7, 1.0)
    ids = np.stack([np.array([rng.choice(V, p=sp_softmax(zq[b, i].astype(np.float64) / temps[b]))
                              for i in range(k)]) for b in range(B)]).astype(np.int32)
    bad = rng.integers(0, k, size=B)
    for b in range(0, B, 2):
        ids[b, bad[b]] = V + 5 if b % 4 == 0 else -1    # rejected there, with p = q
    inp = workloads.make_logits_verify_inputs(71, zp, zq, temps)
    u = OL.uniforms_with_margin(zp, zq, ids, inp.uniforms.numpy(), temps, np.random.default_rng(72))
    ws = vap.verify_logits_workspace(B, k, V, DEV)
    ref = _compare(zp, zq, ids, u, temps, f"empty residual V={V}", workspace=ws)
    assert np.all(ref[1][0::2] <= bad[0::2]) and np.any(ref[1][0::2] == bad[0::2])
    assert vap.get_device_error(ws, clear=True) & vap.DERR_DRAFT_ID
    assert vap.get_device_error(ws) == 0


def test_one_buffer_with_changing_workspace_sizes():
    """Each call passes exactly the bytes its own shape needs, so where the tickets lie moves
    from call to call over data earlier calls left behind: bit-exact every time."""
    lib = vap.load_library()
    shapes = [(16, 4, 128256), (2, 1, 5000), (64, 4, 32000), (1, 0, 7), (3, 12, 4099), (16, 4, 128256), (40, 2, 1000)]
    buf = torch.zeros(max(lib.vap_verify_logits_workspace_bytes(*s) for s in shapes), dtype=torch.uint8, device=DEV)
    for i, (B, k, V) in enumerate(shapes):
        rng = np.random.default_rng(300 + i)
        zp = (2.5 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
        zq = (zp[:, :k] + 0.6 * rng.standard_normal((B, k, V))).astype(np.float32)
        temps = rng.choice([0.0, 0.8, 1.0], size=B)
        inp = workloads.make_logits_verify_inputs(400 + i, zp, zq, temps)
        nbytes = lib.vap_verify_logits_workspace_bytes(B, k, V)
        print("workspace bytes", nbytes, (B, k, V), flush=True)
        _compare(*_margin(inp, 20 + i), f"call {i} {(B, k, V)}", workspace=buf[:nbytes])
    assert vap.get_device_error(buf) == 0


def test_greedy_argmax_ties_pick_the_first_index():
    """Greedy rows whose maximum appears several times: in one lane, across lanes of one
    statistics chunk, and across chunks (2048 tokens each) and verification workgroups.  The
    argmax is the smallest such index (the oracle's reading, np.argmax), so a draft at a later
    tied position is rejected and the emitted token is the first tied index; the sampled
    sequence checks that the ties leave the row statistics right."""
    rng = np.random.default_rng(31)
    B, k, V = 5, 3, 3 * 2048 + 777
    zp = rng.uniform(-1.0, 1.0, (B, k + 1, V)).astype(np.float32)
    zq = rng.uniform(-1.0, 1.0, (B, k, V)).astype(np.float32)
    first = np.zeros((B, k + 1), dtype=np.int64)
    later = np.zeros((B, k + 1), dtype=np.int64)
    for b in range(B):
        for i in range(k + 1):
            f = int(rng.integers(0, V // 2))
            ties = sorted({f, f + 1, f + 64 * int(rng.integers(1, 8)), f + 2048, V - 1 - int(rng.integers(0, 300))})
            zp[b, i, ties] = 4.0
            first[b, i], later[b, i] = ties[0], ties[int(rng.integers(1, len(ties)))]
    temps = np.array([0.0, 0.0, 0.0, 0.0, 1.0])
    inp = workloads.make_logits_verify_inputs(41, zp, zq, temps)
    ids = inp.draft_ids.numpy().copy()
    ids[0] = first[0, :k]                                  # all accepted: bonus = first argmax of row k
    ids[1] = [later[1, 0], first[1, 1], first[1, 2]]       # a later tie is rejected at once
    ids[2] = [first[2, 0], first[2, 1], later[2, 2]]       # rejected at the last draft
    ids[3] = [first[3, 0], later[3, 1], first[3, 2]]
    inp = workloads.LogitsVerifyInputs(**{**inp.__dict__, "draft_ids": torch.as_tensor(ids)})
    zp_, zq_, ids_, u, T = _margin(inp, 8)
    ref = _compare(zp_, zq_, ids_, u, T, "argmax ties")
    assert list(ref[1][:4]) == [3, 0, 2, 1]
    assert ref[0][0, 3] == first[0, 3] and ref[0][1, 0] == first[1, 0] and ref[0][2, 2] == first[2, 2]


def test_batch_above_the_lds_temperature_stage():
    """4100 sequences: above the 4096 temperatures the statistics kernel stages in LDS, so it
    reads each item's temperature from global memory; mixed temperatures, bit-exact."""
    rng = np.random.default_rng(4100)
    B, k, V = 4100, 2, 96
    zp = (2.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    zq = (zp[:, :k] + 0.6 * rng.standard_normal((B, k, V))).astype(np.float32)
    temps = rng.choice([0.0, 0.5, 1.0, 1.7], size=B)
    inp = workloads.make_logits_verify_inputs(4100, zp, zq, temps)
    _compare(*_margin(inp, 41), "B=4100")
