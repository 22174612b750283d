"""The seeded input generators: determinism, distributions, placement and poison."""

import math

import numpy as np
import torch

import workloads as W


def test_lengths_are_deterministic_and_within_recipe():
    for name in W.CONFIG_NAMES:
        L1, Q1, shape = W.config_lengths(name)
        L2, Q2, _ = W.config_lengths(name)
        assert np.array_equal(L1, L2) and np.array_equal(Q1, Q2)
        Hq, Hkv, D, bs, max_ctx = shape
        assert np.all(Q1 >= 1) and np.all(L1 >= Q1) and np.all(L1 <= max_ctx)
    L, Q, _ = W.config_lengths("llama3_8b_decode")
    assert L.size == 64 and L.min() >= 16 and L.max() <= 8192 and np.all(Q == 1)
    assert 300 < np.median(L) < 3000
    L, Q, _ = W.config_lengths("spec_verify_step")
    assert np.all(Q == 5) and L.min() >= 512 and L.max() <= 4096
    L, Q, _ = W.config_lengths("llama70b_share")
    assert L.size == 256 and L.min() >= 128 and L.max() <= 32768
    L, Q, _ = W.config_lengths("mixed_step")
    assert sorted(np.unique(Q).tolist()) == [1, 5, 256]
    assert (Q == 1).sum() == 128 and (Q == 5).sum() == 32 and (Q == 256).sum() == 4


def test_pareto_tail_over_seeds():
    # alpha = 1.5, min 128: median 128 * 2^(1/1.5) ~ 203
    med = [np.median(W.config_lengths("llama70b_share", seed=s)[0]) for s in range(5)]
    assert all(150 < m < 260 for m in med)


def test_tiny_inputs_layout_and_poison():
    a = W.attention_config("tiny")
    a2 = W.attention_config("tiny")
    assert torch.equal(a.q, a2.q) and torch.equal(a.block_tables, a2.block_tables)
    assert torch.equal(torch.isnan(a.kv_pool), torch.isnan(a2.kv_pool))
    assert a.kv_pool.shape == (2, 35, 16, 2, 64) and a.q.shape == (4, 8, 64)
    tables = a.block_tables.numpy()
    L = a.ctx_lens.numpy()
    used = []
    for s in range(4):
        nb = math.ceil(L[s] / 16)
        assert np.all(tables[s, :nb] >= 0) and np.all(tables[s, nb:] == -1)
        used += tables[s, :nb].tolist()
        last = tables[s, nb - 1]
        tail = L[s] % 16
        pool_last = a.kv_pool[:, last]
        if tail:
            assert torch.isnan(pool_last[:, tail:]).all()
            assert torch.isfinite(pool_last[:, :tail]).all()
        for b in tables[s, :nb - 1]:
            assert torch.isfinite(a.kv_pool[:, b]).all()
    assert len(set(used)) == len(used) == 29
    unused = sorted(set(range(35)) - set(used))
    assert torch.isnan(a.kv_pool[:, unused]).all()


def test_verify_inputs_shapes_and_uniforms():
    v = W.verify_config("tiny")
    assert v.p.shape == (4, 5, 1000) and v.q.shape == (4, 4, 1000)
    assert v.draft_ids.dtype == torch.int32 and v.uniforms.dtype == torch.float32
    u = v.uniforms.numpy()
    assert np.all(u > 0) and np.all(u < 1)
    np.testing.assert_allclose(v.p.sum(-1).numpy(), 1.0, atol=1e-5)
    assert np.all((v.draft_ids.numpy() >= 0) & (v.draft_ids.numpy() < 1000))
    v2 = W.verify_config("tiny")
    assert torch.equal(v.p, v2.p) and torch.equal(v.draft_ids, v2.draft_ids)
    assert torch.equal(v.uniforms, v2.uniforms)


def test_u8_inputs_share_lengths_and_tables_and_poison_scales_only():
    a = W.attention_config("tiny")
    b = W.attention_config("tiny", kv_format="u8")
    assert torch.equal(a.ctx_lens, b.ctx_lens) and torch.equal(a.q_lens, b.q_lens)
    assert torch.equal(a.q, b.q)                       # q is drawn before the pool
    assert b.kv_pool.dtype == torch.uint8 and b.kv_pool.shape == a.kv_pool.shape
    NB, bs, Hkv = b.num_blocks, b.block_size, b.num_kv_heads
    assert b.kv_scales.shape == (NB, Hkv, bs, 4) and b.kv_scales.dtype == torch.float32
    sc = b.kv_scales.numpy()
    tables = b.block_tables.numpy()
    owned = np.zeros((NB, bs), bool)
    for s in range(b.num_seqs):
        L = int(b.ctx_lens[s])
        for j in range(L):
            owned[tables[s, j // bs], j % bs] = True
    live = sc.transpose(0, 2, 1, 3)[owned]              # [n_owned, Hkv, 4]
    assert np.isfinite(live).all()
    assert ((live[..., 0] >= 0.01) & (live[..., 0] <= 0.03)).all()
    assert ((live[..., 1] >= 112) & (live[..., 1] <= 143) & (live[..., 1] == np.round(live[..., 1]))).all()
    assert np.isnan(sc.transpose(0, 2, 1, 3)[~owned]).all()
