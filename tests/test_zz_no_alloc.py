"""spec_verify_static -- spec_verify with the library's static device scratch instead of a
workspace (for callers that cannot allocate) -- against spec_verify through the C ABI.

Two calls in a row on the same device scratch, the second with a smaller batch and vocabulary:
ids and counts bit-exact with spec_verify's (and with the oracle, uniforms at least 1e-6 from
every threshold); device errors reach the caller's word; a batch above the scratch's 4096
sequences is refused on the host.
"""

import numpy as np
import pytest
import torch

import verify_attention_paged_amd as vap
import workloads
from oracle import spec_verify as OS

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(B, V, seed):
    rng = np.random.default_rng(seed)
    pl = 3.0 * rng.standard_normal((B, 5, V))
    ql = pl[:, :4] + 0.7 * rng.standard_normal((B, 4, V))
    vin = workloads.make_verify_inputs(seed, p_logits=pl, q_logits=ql, rng=rng)
    p = vin.p.numpy().astype(np.float64)
    q = vin.q.numpy().astype(np.float64)
    ids = vin.draft_ids.numpy()
    u = OS.uniforms_with_margin(p, q, ids, vin.uniforms.numpy(), np.random.default_rng(seed + 1))
    return vin, ids, u


def test_static_scratch_matches_spec_verify_on_two_calls():
    for B, V, seed in [(64, 128256, 501), (16, 32000, 502)]:       # the second call is smaller
        vin, ids, u = _inputs(B, V, seed)
        print("spec_verify_static B", B, "V", V, flush=True)
        p_t, q_t = vin.p.to(DEV), vin.q.to(DEV)
        i_t = torch.as_tensor(ids, dtype=torch.int32, device=DEV)
        u_t = torch.as_tensor(u, dtype=torch.float32, device=DEV)
        out_s = torch.full((B, 5), -7, dtype=torch.int32, device=DEV)
        n_s = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        vap.spec_verify_static(p_t, q_t, i_t, u_t, out_s, n_s, device_error=err)
        out_w, n_w = vap.spec_verify(p_t, q_t, i_t, u_t)             # the workspace entry point
        torch.cuda.synchronize()
        assert torch.equal(out_s, out_w) and torch.equal(n_s, n_w), f"B={B} V={V}"
        ref_out, ref_n = OS.spec_verify(vin.p.numpy().astype(np.float64), vin.q.numpy().astype(np.float64), ids,
                                        u.astype(np.float64))
        assert np.array_equal(out_s.cpu().numpy(), ref_out) and np.array_equal(n_s.cpu().numpy(), ref_n)
        assert int(err.item()) == 0


def test_device_errors_reach_the_callers_word():
    vin, ids, u = _inputs(8, 1000, 503)
    ids = ids.copy()
    ids[3, 0] = 5000                                                # outside the vocabulary
    p_t, q_t = vin.p.to(DEV), vin.q.to(DEV)
    i_t = torch.as_tensor(ids, dtype=torch.int32, device=DEV)
    u_t = torch.as_tensor(u, dtype=torch.float32, device=DEV)
    out_s = torch.empty((8, 5), dtype=torch.int32, device=DEV)
    n_s = torch.empty((8,), dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    vap.spec_verify_static(p_t, q_t, i_t, u_t, out_s, n_s, device_error=err)
    out_w, n_w = vap.spec_verify(p_t, q_t, i_t, u_t)
    torch.cuda.synchronize()
    assert int(err.item()) & vap.DERR_DRAFT_ID
    assert torch.equal(out_s, out_w) and torch.equal(n_s, n_w) and int(n_s[3].item()) == 0


def test_batches_above_the_static_scratch_are_refused():
    B = 4097
    p = torch.full((B, 1, 8), 0.125, dtype=torch.float32, device=DEV)
    u = torch.full((B, 1), 0.5, dtype=torch.float32, device=DEV)
    out = torch.empty((B, 1), dtype=torch.int32, device=DEV)
    n = torch.empty((B,), dtype=torch.int32, device=DEV)
    with pytest.raises(vap.VapError) as e:
        vap.spec_verify_static(p, None, None, u, out, n)
    assert e.value.code == vap._binding.VAP_EINVAL
