"""Pins of the oracle's KV append / commit (CPU only).

* The 8-bit quantiser equals torch's per-channel min/max observer (scale, zero point) and
  torch's per-channel quantiser (codes), bit for bit.
* Append: reading the new positions back through the block table (the oracle's gather, pinned
  with the attention oracle) returns the written rows; every other pool entry is unchanged.
* Commit of a draft tree: after the accepted nodes are moved, a decode row at the committed
  length sees exactly the prefix, the root and the accepted path, so its output equals the
  tree attention of the last accepted node (itself pinned to the causal verify) bit for bit.
* Commit of a chain changes only the lengths (L - Q + 1 + n).
"""

import numpy as np
import pytest
import torch
from torch.ao.quantization.observer import PerChannelMinMaxObserver

import workloads
from oracle import attention as A
from oracle import kv_cache as K


def _torch_quantize(x2d: np.ndarray):
    obs = PerChannelMinMaxObserver(ch_axis=0, dtype=torch.quint8, qscheme=torch.per_channel_affine)
    t = torch.from_numpy(x2d)
    obs(t)
    sc, zp = obs.calculate_qparams()
    codes = torch.quantize_per_channel(t, sc.double(), zp.long(), 0, torch.quint8).int_repr().numpy()
    return codes, sc.numpy().astype(np.float32), zp.numpy().astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantiser_equals_torch_per_channel_minmax(seed):
    rng = np.random.default_rng(seed)
    n, D = 3000, 128
    x = (rng.standard_normal((n, D)) * rng.uniform(0.001, 8, (n, 1)) + rng.uniform(-3, 3, (n, 1))).astype(np.float32)
    x[0] = 0.0                                 # all zero
    x[1] = 2.5                                 # constant positive
    x[2] = -0.75                               # constant negative
    x[3] = np.abs(x[3])                        # one-signed rows
    x[4] = -np.abs(x[4])
    codes, sc, z = K.quantize_rows_u8(x)
    tc, tsc, tz = _torch_quantize(x)
    np.testing.assert_array_equal(sc, tsc)
    np.testing.assert_array_equal(z.view(np.uint32), tz.view(np.uint32))   # integer zero points: +0, never -0
    np.testing.assert_array_equal(codes, tc)
    deq = sc[:, None].astype(np.float64) * (codes.astype(np.float64) - z[:, None])
    assert np.all(np.abs(deq - x) <= 0.5 * sc[:, None].astype(np.float64) * (1 + 1e-5) + 1e-7)


def _batch(seed, fmt="bf16"):
    return workloads.make_attention_inputs(seed, ctx_lens=[20, 64, 100, 33], q_lens=[5, 1, 17, 33],
                                           num_q_heads=8, num_kv_heads=2, head_dim=32, block_size=16,
                                           kv_format=fmt)


def _new_rows(inp, seed):
    g = torch.Generator().manual_seed(seed)
    T = inp.total_q
    shape = (T, inp.num_kv_heads, inp.head_dim)
    return (torch.randn(shape, generator=g).to(torch.bfloat16), torch.randn(shape, generator=g).to(torch.bfloat16))


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_append_writes_exactly_the_new_positions():
    inp = _batch(3)
    k, v = _new_rows(inp, 4)
    pool = _bits(inp.kv_pool)
    out = K.kv_append(pool, inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy(), _bits(k), _bits(v))
    touched = np.zeros(out.shape[1:3], bool)
    row = 0
    for s in range(inp.num_seqs):
        L, Q = int(inp.ctx_lens[s]), int(inp.q_lens[s])
        got_k = A.gather_sequence_kv(out[0], inp.block_tables[s].numpy(), L)[L - Q:]
        got_v = A.gather_sequence_kv(out[1], inp.block_tables[s].numpy(), L)[L - Q:]
        np.testing.assert_array_equal(got_k, _bits(k)[row:row + Q])
        np.testing.assert_array_equal(got_v, _bits(v)[row:row + Q])
        slots = A.physical_slots(inp.block_tables[s].numpy(), L, inp.block_size)[L - Q:]
        touched.reshape(-1)[slots] = True
        row += Q
    same = (out == pool) | (np.isnan(A.bf16_bits_to_f64(out)) & np.isnan(A.bf16_bits_to_f64(pool)))
    assert same[:, ~touched].all()


def test_append_u8_quantises_each_row_and_touches_nothing_else():
    inp = _batch(5, "u8")
    k, v = _new_rows(inp, 6)
    kf, vf = k.float().numpy(), v.float().numpy()
    codes, scales = K.kv_append_u8(inp.kv_pool.numpy(), inp.kv_scales.numpy(), inp.block_tables.numpy(),
                                   inp.ctx_lens.numpy(), inp.q_lens.numpy(), kf, vf)
    row = 0
    for s in range(inp.num_seqs):
        L, Q = int(inp.ctx_lens[s]), int(inp.q_lens[s])
        kk, vv = A.gather_sequence_kv_u8(codes, scales, inp.block_tables[s].numpy(), L)
        for got, x in ((kk[L - Q:], kf[row:row + Q]), (vv[L - Q:], vf[row:row + Q])):
            c, sc, z = _torch_quantize(x.reshape(-1, x.shape[-1]))
            ref = sc[:, None].astype(np.float64) * (c.astype(np.float64) - z[:, None])
            np.testing.assert_array_equal(got.reshape(-1, x.shape[-1]), ref)
        row += Q
    # untouched slots keep codes and scales (NaN poison included)
    assert (codes == inp.kv_pool.numpy()).mean() > 0.5
    old = inp.kv_scales.numpy()
    same = (scales == old) | (np.isnan(scales) & np.isnan(old))
    assert same.mean() > 0.5


def test_chain_commit_only_shortens():
    inp = _batch(7)
    n = np.array([2, 0, 16, 5])
    pool = _bits(inp.kv_pool)
    chain = np.array([np.arange(1, 40) for _ in range(inp.num_seqs)])
    out, _, L2 = K.kv_commit_tree(pool, inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy(), chain, n)
    np.testing.assert_array_equal(L2, inp.ctx_lens.numpy() - inp.q_lens.numpy() + 1 + n)
    same = (out == pool) | (np.isnan(A.bf16_bits_to_f64(out)) & np.isnan(A.bf16_bits_to_f64(pool)))
    assert same.all()


@pytest.mark.parametrize("fmt", ["bf16", "u8"])
def test_tree_commit_then_decode_equals_tree_attention_of_the_last_node(fmt):
    rng = np.random.default_rng(11)
    sizes = [9, 16, 5]
    inp = workloads.make_attention_inputs(12, ctx_lens=[40, 100, 20], q_lens=sizes, num_q_heads=8, num_kv_heads=2,
                                          head_dim=32, block_size=16, kv_format=fmt)
    parents = [workloads.random_tree_parents(rng, n) for n in sizes]
    masks = np.concatenate([workloads.tree_masks(p) for p in parents])
    qb = _bits(inp.q)
    tables, L, Q = inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy()
    # an accepted path per sequence: walk down from the root through the first child
    paths, n_acc = [], []
    for p in parents:
        path, u = [], 0
        while True:
            kids = [c for c in range(len(p)) if p[c] == u]
            if not kids or len(path) >= 3:
                break
            u = kids[-1]
            path.append(u)
        paths.append(path + [-1] * (20 - len(path)))
        n_acc.append(len(path))
    n_acc = np.array(n_acc)
    starts = np.concatenate([[0], np.cumsum(Q)])
    if fmt == "bf16":
        pool = _bits(inp.kv_pool)
        tree = A.paged_attention_bf16(qb, pool, tables, L, Q, tree_mask=masks)
        pool2, _, L2 = K.kv_commit_tree(pool, tables, L, Q, np.array(paths), n_acc)
    else:
        tree = A.paged_attention_u8(qb, inp.kv_pool.numpy(), inp.kv_scales.numpy(), tables, L, Q, tree_mask=masks)
        codes2, scales2, L2 = K.kv_commit_tree(inp.kv_pool.numpy(), tables, L, Q, np.array(paths), n_acc,
                                               kv_scales=inp.kv_scales.numpy())
    for s in range(len(sizes)):
        last = paths[s][n_acc[s] - 1] if n_acc[s] else 0
        t = int(starts[s] + last)
        q1 = qb[t:t + 1]
        args = (tables[s:s + 1], np.array([L2[s]]), np.array([1]))
        if fmt == "bf16":
            dec = A.paged_attention_bf16(q1, pool2, *args)
        else:
            dec = A.paged_attention_u8(q1, codes2, scales2, *args)
        for h in range(inp.num_q_heads):
            np.testing.assert_array_equal(dec[(0, h)], tree[(t, h)])
