"""Pins of the oracle's tree-masked attention (CPU only).

* A chain (every node's parent is the previous node) is the causal verify: bit-identical.
* Path equivalence: node i of a tree sees the prefix and its root-to-i path, so its output equals
  the causal verify of a sequence whose new rows are exactly that path (K/V of the path nodes
  laid out contiguously after the prefix) -- bit-identical, through the already pinned causal
  path.
* A one-node tree is a decode row.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A


def _bits(t):
    return t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)


def _path(parents, i):
    p = []
    while i >= 0:
        p.append(i)
        i = int(parents[i])
    return p[::-1]


@pytest.mark.parametrize("Q", [1, 2, 5, 17])
def test_chain_mask_is_the_causal_verify(Q):
    rng = np.random.default_rng(Q)
    L = Q + int(rng.integers(0, 60))
    q = rng.standard_normal((Q, 8, 32))
    k = rng.standard_normal((L, 2, 32))
    v = rng.standard_normal((L, 2, 32))
    chain = workloads.tree_masks(np.arange(Q) - 1)
    a = A.attention_sequence(q, k, v)
    b = A.attention_sequence(q, k, v, tree_mask=chain)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_each_node_equals_the_causal_verify_of_its_path(seed):
    rng = np.random.default_rng(100 + seed)
    Q = int(rng.integers(2, 40))
    prefix = int(rng.integers(0, 50))
    L = prefix + Q
    Hq, Hkv, D = 6, 3, 16
    parents = workloads.random_tree_parents(rng, Q)
    masks = workloads.tree_masks(parents)
    q = rng.standard_normal((Q, Hq, D))
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    tree = A.attention_sequence(q, k, v, tree_mask=masks)
    for i in range(Q):
        path = _path(parents, i)
        keys = np.concatenate([np.arange(prefix), prefix + np.array(path)])
        chain = A.attention_sequence(q[path], k[keys], v[keys])
        np.testing.assert_array_equal(tree[i], chain[-1])


def test_single_node_tree_is_a_decode_row():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 4, 16))
    k = rng.standard_normal((30, 2, 16))
    v = rng.standard_normal((30, 2, 16))
    np.testing.assert_array_equal(A.attention_sequence(q, k, v),
                                  A.attention_sequence(q, k, v, tree_mask=np.array([1])))


def test_paged_tree_config_matches_path_equivalence():
    """The paged entry point with the tree_verify_step recipe (a few sequences checked)."""
    inp = workloads.attention_config("tree_verify_step")
    qb, pool = _bits(inp.q), _bits(inp.kv_pool)
    tables, L, Q = inp.block_tables.numpy(), inp.ctx_lens.numpy(), inp.q_lens.numpy()
    masks = inp.tree_mask.numpy()
    starts = np.concatenate([[0], np.cumsum(Q)])
    for s in (0, 7):
        rows = [(int(starts[s] + i), h) for i in range(int(Q[s])) for h in (0, 13)]
        got = A.paged_attention_bf16(qb, pool, tables, L, Q, rows=rows, tree_mask=masks)
        ks = A.bf16_bits_to_f64(A.gather_sequence_kv(pool[0], tables[s], int(L[s])))
        vs = A.bf16_bits_to_f64(A.gather_sequence_kv(pool[1], tables[s], int(L[s])))
        qs = A.bf16_bits_to_f64(qb[starts[s]:starts[s] + Q[s]])
        m = masks[starts[s]:starts[s] + Q[s]].view(np.uint64)
        prefix = int(L[s] - Q[s])
        for i in range(int(Q[s])):
            path = [j for j in range(int(Q[s])) if (int(m[i]) >> j) & 1]
            keys = np.concatenate([np.arange(prefix), prefix + np.array(path)])
            chain = A.attention_sequence(qs[path], ks[keys], vs[keys])
            for h in (0, 13):
                np.testing.assert_array_equal(got[(int(starts[s] + i), h)], chain[-1, h])
