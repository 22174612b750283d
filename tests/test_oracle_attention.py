"""Pins for the attention oracle (CPU only).

Each test checks ``oracle.attention`` against something other than itself: hand-worked closed
forms (tests/golden), torch's fp64 scaled_dot_product_attention with an explicit mask, exact
special cases, and invariants that paging and causal verification fix.  Together they catch a
dropped max-shift, a wrong scale, an off-by-one causal limit, a wrong GQA head mapping, a
transposed operand and a wrong block-table translation.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa_reference(q_seq, k_seq, v_seq, scale=None):
    """torch fp64 SDPA with KV heads repeated per group and an explicit causal-suffix mask."""
    Q, Hq, D = q_seq.shape
    L, Hkv, _ = k_seq.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q_seq).permute(1, 0, 2)                       # [Hq, Q, D]
    kt = torch.from_numpy(k_seq).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(v_seq).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
    i = torch.arange(Q)[:, None]
    j = torch.arange(L)[None, :]
    mask = j <= (L - Q + i)                                              # True = may attend
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_golden_worked_cases(golden_dir):
    with open(os.path.join(golden_dir, "attention_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        out = A.attention_sequence(q, k, v, c["scale"])
        np.testing.assert_allclose(out, np.array(c["out"]), rtol=1e-12, atol=1e-12, err_msg=c["name"])


def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    q, k, v = _rand(rng, 1, 8, 64), _rand(rng, 1, 2, 64), _rand(rng, 1, 2, 64)
    out = A.attention_sequence(q, k, v)
    for h in range(8):
        assert np.array_equal(out[0, h], v[0, h // 4])


def test_equal_keys_give_the_mean_of_visible_values():
    rng = np.random.default_rng(1)
    L, Q = 37, 5
    k = np.broadcast_to(_rand(rng, 1, 1, 16), (L, 1, 16)).copy()
    v = _rand(rng, L, 1, 16)
    q = _rand(rng, Q, 3, 16)
    out = A.attention_sequence(q, k, v)
    for i in range(Q):
        visible = L - Q + i + 1
        np.testing.assert_allclose(out[i, 0], v[:visible, 0].mean(axis=0), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("Q,L,Hq,Hkv,D", [(1, 1, 4, 4, 8), (1, 50, 8, 8, 64), (5, 40, 4, 4, 32),
                                          (5, 5, 2, 2, 16), (17, 30, 6, 6, 8), (1, 33, 32, 8, 128),
                                          (5, 77, 32, 8, 128), (3, 19, 8, 1, 64)])
def test_matches_torch_sdpa_fp64(Q, L, Hq, Hkv, D):
    rng = np.random.default_rng(Q * 1000 + L)
    q, k, v = _rand(rng, Q, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    np.testing.assert_allclose(A.attention_sequence(q, k, v), _sdpa_reference(q, k, v),
                               rtol=1e-11, atol=1e-12)


def test_matches_torch_sdpa_with_explicit_scale_and_large_scores():
    """Scores of magnitude ~1e3 overflow exp() unless the maximum is subtracted first."""
    rng = np.random.default_rng(7)
    q, k, v = 40.0 * _rand(rng, 3, 4, 32), 40.0 * _rand(rng, 25, 2, 32), _rand(rng, 25, 2, 32)
    for scale in (None, 0.3):
        out = A.attention_sequence(q, k, v, scale)
        assert np.all(np.isfinite(out))
        np.testing.assert_allclose(out, _sdpa_reference(q, k, v, scale), rtol=1e-10, atol=1e-12)


def test_verify_rows_equal_sequential_decodes():
    """Row i of a q_len = k+1 call equals a single-row decode over the first L-(Q-1-i) keys."""
    rng = np.random.default_rng(3)
    Q, L, Hq, Hkv, D = 5, 23, 8, 2, 16
    q, k, v = _rand(rng, Q, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    full = A.attention_sequence(q, k, v)
    for i in range(Q):
        Lp = L - (Q - 1 - i)
        one = A.attention_sequence(q[i:i + 1], k[:Lp], v[:Lp])
        assert np.array_equal(one[0], full[i])


def _scatter(k_seqs, v_seqs, bs, rng, extra_blocks=3):
    """Place contiguous per-sequence KV at random pool blocks; return pool and tables."""
    nblk = [(x.shape[0] + bs - 1) // bs for x in k_seqs]
    NB = sum(nblk) + extra_blocks
    Hkv, D = k_seqs[0].shape[1:]
    pool = np.full((2, NB, bs, Hkv, D), np.nan)
    perm = rng.permutation(NB)
    tables = np.full((len(k_seqs), max(nblk)), -1, dtype=np.int64)
    c = 0
    for s, (ks, vs) in enumerate(zip(k_seqs, v_seqs)):
        for b in range(nblk[s]):
            phys = perm[c]
            c += 1
            tables[s, b] = phys
            rows = ks[b * bs:(b + 1) * bs]
            pool[0, phys, :rows.shape[0]] = rows
            pool[1, phys, :rows.shape[0]] = vs[b * bs:(b + 1) * bs]
    return pool, tables


@pytest.mark.parametrize("bs", [16, 32])
def test_block_table_permutation_gives_contiguous_result_bit_exact(bs):
    rng = np.random.default_rng(bs)
    Ls, Qs = [1, 15, 16, 17, 40, 64], [1, 1, 5, 5, 1, 5]
    Hq, Hkv, D = 8, 2, 32
    ks = [_rand(rng, L, Hkv, D) for L in Ls]
    vs = [_rand(rng, L, Hkv, D) for L in Ls]
    q = _rand(rng, sum(Qs), Hq, D)
    expect = []
    r = 0
    for s in range(len(Ls)):
        expect.append(A.attention_sequence(q[r:r + Qs[s]], ks[s], vs[s]))
        r += Qs[s]
    expect = np.concatenate(expect)
    for trial in range(3):
        pool, tables = _scatter(ks, vs, bs, rng)
        out = A.paged_attention(q, pool[0], pool[1], tables, Ls, Qs)
        assert np.array_equal(out, expect)          # NaN-poisoned unused rows never read


def test_shared_prefix_blocks():
    """Two tables sharing their first physical blocks see the same prefix KV."""
    rng = np.random.default_rng(11)
    bs, Hq, Hkv, D = 16, 4, 2, 16
    pool = _rand(rng, 2, 20, bs, Hkv, D)
    shared = [3, 7, 1, 12]                       # 64 shared tokens
    tables = np.array([shared + [5, 9], shared + [0, 18]])
    L = [64 + 20, 64 + 20]
    q = np.repeat(_rand(rng, 1, Hq, D), 2, axis=0)
    out = A.paged_attention(q, pool[0], pool[1], tables, L, [1, 1])
    # the two sequences differ only after the shared prefix: check each against its own gather
    for s in range(2):
        ks = np.concatenate([pool[0, b] for b in tables[s]])[:L[s]]
        vs = np.concatenate([pool[1, b] for b in tables[s]])[:L[s]]
        assert np.array_equal(out[s], A.attention_sequence(q[s:s + 1], ks, vs)[0])
    # identical tables and queries -> identical outputs
    tables2 = np.array([shared + [5, 9], shared + [5, 9]])
    out2 = A.paged_attention(q, pool[0], pool[1], tables2, [70, 70], [1, 1])
    assert np.array_equal(out2[0], out2[1])


def test_physical_slot_translation_by_hand():
    table = np.array([4, 0, 2])
    slots = A.physical_slots(table, 7, 3)
    assert slots.tolist() == [12, 13, 14, 0, 1, 2, 6]
    with pytest.raises(ValueError):
        A.physical_slots(np.array([1, -1]), 5, 4)


def test_bf16_bits_conversion():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x4049, 0x3EAB],
                    dtype=np.uint16)
    got = A.bf16_bits_to_f64(bits)
    expect = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133, 3.140625, 0.333984375]
    assert got.tolist() == expect
    # every finite pattern agrees with torch's exact bf16 -> fp64 conversion
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(allbits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = A.bf16_bits_to_f64(allbits)
    ok = np.isfinite(t)
    assert np.array_equal(mine[ok], t[ok])
    assert np.array_equal(np.isnan(mine), np.isnan(t))


def test_bf16_entry_point_agrees_with_float_entry_point():
    import workloads
    inp = workloads.attention_config("tiny")
    q_bits = inp.q.view(torch.int16).numpy().view(np.uint16)
    pool_bits = inp.kv_pool.view(torch.int16).numpy().view(np.uint16)
    tables = inp.block_tables.numpy()
    L, Q = inp.ctx_lens.numpy(), inp.q_lens.numpy()
    full = A.paged_attention_bf16(q_bits, pool_bits, tables, L, Q)
    q64 = inp.q.to(torch.float64).numpy()
    p64 = inp.kv_pool.to(torch.float64).numpy()
    ref = A.paged_attention(q64, p64[0], p64[1], tables, L, Q)
    for (t, h), o in full.items():
        assert np.array_equal(o, ref[t, h])
        assert np.all(np.isfinite(o))
    some = [(0, 3), (2, 7), (3, 0)]
    sub = A.paged_attention_bf16(q_bits, pool_bits, tables, L, Q, rows=some)
    assert set(sub) == set(some)
    for key in some:
        assert np.array_equal(sub[key], full[key])


def test_rejects_bad_shapes():
    rng = np.random.default_rng(0)
    with pytest.raises(ValueError):
        A.attention_sequence(_rand(rng, 1, 3, 4), _rand(rng, 2, 2, 4), _rand(rng, 2, 2, 4))
    with pytest.raises(ValueError):
        A.attention_sequence(_rand(rng, 3, 2, 4), _rand(rng, 2, 2, 4), _rand(rng, 2, 2, 4))
