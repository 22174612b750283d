"""Seeded random shapes through paged_attn_step and spec_verify, each against the oracle.

Attention: random KV-head counts, group sizes, head dims, block sizes and cache formats (bf16,
INT8, FP8), with decode, verify, prefill-chunk and mixed length mixes, so units of one, two and
four row tiles, masked tails and split units all occur; bar |gpu - oracle| <= 2e-3 + 1e-2
|oracle| on every (row, head).  Verification: random vocabularies, draft counts and batch sizes,
ids and counts bit-exact with uniforms placed at least 1e-6 from every threshold.
"""

import numpy as np
import pytest
import torch

import verify_attention_paged_amd as vap
import workloads
from oracle import spec_verify as OS
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _attention_case(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if g * Hkv <= 32]))
    D, bs = int(rng.choice([64, 128])), int(rng.choice([16, 32]))
    fmt = str(rng.choice(["bf16", "bf16", "u8", "fp8"]))
    kind = str(rng.choice(["decode", "verify", "mixed", "prefill"]))
    B = int(rng.integers(1, 24 if kind in ("decode", "verify") else 10))
    ql = []
    for _ in range(B):
        if kind == "decode":
            ql.append(1)
        elif kind == "verify":
            ql.append(int(rng.integers(1, 9)))
        elif kind == "prefill":
            ql.append(int(rng.integers(8, 65)))
        else:
            ql.append(int(rng.choice([1, 1, 5, int(rng.integers(8, 65))])))
    ctx = [int(max(q, rng.integers(1, 2500))) for q in ql]
    inp = workloads.make_attention_inputs(seed, ctx_lens=ctx, q_lens=ql, num_q_heads=G * Hkv, num_kv_heads=Hkv,
                                          head_dim=D, block_size=bs, kv_format=fmt)
    return inp, f"seed {seed}: {kind} B {B} Hq {G * Hkv} Hkv {Hkv} D {D} bs {bs} {fmt}"


@pytest.mark.parametrize("seed", range(7000, 7024))
def test_random_attention_shapes(seed):
    inp, what = _attention_case(seed)
    print(what, flush=True)
    ref = H.oracle_rows(inp)                 # on the CPU, before the GPU call
    out = vap.paged_attn_step(**H.to_device(inp))
    torch.cuda.synchronize()
    H.assert_close_rows(out, ref, what)


@pytest.mark.parametrize("seed", range(12))
def test_random_verification_shapes(seed):
    rng = np.random.default_rng(10_000 + seed)
    V = int(rng.choice([1000, 4099, 32000, 128256]))
    k = int(rng.integers(0, 7))
    B = int(rng.choice([1, 3, 16])) if V == 128256 else int(rng.choice([1, 3, 16, 40, 130]))
    zl = rng.normal(0.0, float(rng.choice([1.0, 3.0, 6.0])), (B, k + 1, V))
    ql = zl[:, :k] + rng.normal(0.0, float(rng.choice([0.1, 0.7, 2.0])), (B, k, V))
    vin = workloads.make_verify_inputs(seed, p_logits=zl, q_logits=ql)
    p64, q64, ids = vin.p.numpy().astype(np.float64), vin.q.numpy().astype(np.float64), vin.draft_ids.numpy()
    u = OS.uniforms_with_margin(p64, q64, ids, vin.uniforms.numpy(), np.random.default_rng(seed))
    what = f"seed {seed}: B {B} k {k} V {V}"
    print(what, flush=True)
    ref_ids, ref_n = OS.spec_verify(p64, q64, ids, u.astype(np.float64))
    out_ids, n = vap.spec_verify(vin.p.to(DEV), vin.q.to(DEV), vin.draft_ids.to(DEV),
                                 torch.as_tensor(np.ascontiguousarray(u, dtype=np.float32), device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(n.cpu().numpy(), ref_n), f"{what}: n_accepted {n.cpu().numpy()} vs {ref_n}"
    assert np.array_equal(out_ids.cpu().numpy(), ref_ids), f"{what}: ids differ"
