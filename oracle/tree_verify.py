"""Oracle: verification of a draft token tree, sequential and in float64 (test infrastructure).

The pages describe modified rejection sampling for a chain of drafts [P4 §"The Modified
Rejection Sampling Algorithm"] and say that tree variants draft several candidates per position
and verify the whole token tree in one pass [P4 §"4. Tree Attention & Medusa Heads"; P3
§"Draft Model Selection and Tree-Style Variants"], without spelling out the acceptance rule.
Reading taken (the plainest extension of the chain rule, the one that stays lossless when a
node's children are independent draws from that node's draft distribution):

* The tree has N nodes in an order where parents come first; node 0 is the last committed token
  (the root), node i > 0 holds draft token x_i.  p[u] is the target's next-token distribution
  after node u; q[u] is the draft distribution u's children were drawn from.
* Start at the root with the current target distribution p_cur = p[0].  Test u's children in
  index order with the chain rule: child c passes when r_c <= min(1, p_cur(x_c) / q[u](x_c)).
  After each rejection p_cur becomes the normalised residual max(0, p_cur - q[u]) / Z (kept as
  it is when Z = 0).  The first child that passes is accepted: emit x_c, move to c, and reset
  p_cur = p[c].
* When the current node has no child left to test (all rejected, or it is a leaf), draw one
  token from p_cur by the same inverse CDF as the chain verifier, with the uniform u_0, and stop.
  For a chain this is exactly the chain verifier (residual after a rejection, bonus row at the
  end of the path).

Uniforms: one per node; u_i (i > 0) is the accept test of node i, u_0 the final draw.  Decision
details (exact accept test, inverse CDF, Z = 0, out-of-range ids) are those of
``oracle.spec_verify``.
"""

from __future__ import annotations

import numpy as np

from .spec_verify import accept_draft, sample_inverse_cdf


def tree_children(parents) -> list:
    """Children of every node, in increasing index."""
    par = np.asarray(parents, dtype=np.int64)
    kids = [[] for _ in range(par.size)]
    for i in range(1, par.size):
        kids[int(par[i])].append(i)
    return kids


def residual(p_cur: np.ndarray, q_row: np.ndarray) -> np.ndarray:
    """max(0, p_cur - q_row) normalised by its (left-to-right fp64) sum; p_cur if the sum is 0."""
    w = np.maximum(0.0, np.asarray(p_cur, np.float64) - np.asarray(q_row, np.float64))
    Z = 0.0
    for x in range(w.size):
        Z += w[x]
    return w / Z if Z > 0.0 else np.asarray(p_cur, np.float64)


def tree_verify_sequence(p_rows, q_rows, parents, tokens, uniforms):
    """One sequence.  p_rows, q_rows [N, V]; parents, tokens, uniforms [N].

    Returns (out_ids [N]: accepted tokens then the drawn token, -1 after; path [N]: accepted
    node indices, -1 after; n_accepted).
    """
    p_rows = np.asarray(p_rows, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    N, V = p_rows.shape
    kids = tree_children(parents)
    ids, path = [], []
    u = 0
    p_cur = p_rows[0]
    while True:
        accepted = None
        for c in kids[u]:
            x = int(tokens[c])
            inside = 0 <= x < V
            P = p_cur[x] if inside else 0.0
            Qx = q_rows[u, x] if inside else 0.0
            if accept_draft(P, Qx, uniforms[c]):
                accepted = c
                break
            p_cur = residual(p_cur, q_rows[u])
        if accepted is None:
            y = sample_inverse_cdf(p_cur, uniforms[0])
            ids.append(max(y, 0))
            break
        path.append(accepted)
        ids.append(int(tokens[accepted]))
        u = accepted
        p_cur = p_rows[u]
    out = np.full(N, -1, dtype=np.int64)
    out[:len(ids)] = ids
    nodes = np.full(N, -1, dtype=np.int64)
    nodes[:len(path)] = path
    return out, nodes, len(path)


def tree_verify(p, q, parents, tokens, uniforms):
    """Batch wrapper over [B, N, V] rows and [B, N] trees; returns (out_ids, path, n_accepted)."""
    B, N = np.asarray(parents).shape
    out = np.empty((B, N), dtype=np.int64)
    nodes = np.empty((B, N), dtype=np.int64)
    n = np.empty(B, dtype=np.int64)
    for b in range(B):
        out[b], nodes[b], n[b] = tree_verify_sequence(p[b], q[b], parents[b], tokens[b], uniforms[b])
    return out, nodes, n


# ----------------------------------------------------------------------------------------
# decision margins (test harness): every threshold the walk evaluates, so that uniforms can
# be placed away from them and summation order cannot flip a decision.
# ----------------------------------------------------------------------------------------

def tree_decision_margin(p_rows, q_rows, parents, tokens, uniforms) -> float:
    p_rows = np.asarray(p_rows, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    N, V = p_rows.shape
    kids = tree_children(parents)
    margin = np.inf
    u = 0
    p_cur = p_rows[0]
    while True:
        accepted = None
        for c in kids[u]:
            x = int(tokens[c])
            inside = 0 <= x < V
            P = p_cur[x] if inside else 0.0
            Qx = q_rows[u, x] if inside else 0.0
            if Qx > 0.0:
                margin = min(margin, abs(float(uniforms[c]) - min(1.0, P / Qx)))
            if accept_draft(P, Qx, uniforms[c]):
                accepted = c
                break
            p_cur = residual(p_cur, q_rows[u])
        if accepted is None:
            cum = np.cumsum(p_cur)
            if cum[-1] > 0.0:
                margin = min(margin, float(np.min(np.abs(float(uniforms[0]) - cum / cum[-1]))))
            return margin
        u = accepted
        p_cur = p_rows[u]


def tree_uniforms_with_margin(p, q, parents, tokens, uniforms, rng: np.random.Generator,
                              eps: float = 1e-6, max_tries: int = 1000) -> np.ndarray:
    """Redraw (seeded) every sequence's uniforms until its decision margin is >= eps."""
    u = np.array(uniforms, dtype=np.float32, copy=True)
    for b in range(u.shape[0]):
        for _ in range(max_tries):
            if tree_decision_margin(p[b], q[b], parents[b], tokens[b], u[b]) >= eps:
                break
            j = rng.integers(0, 1 << 24, size=u.shape[1], dtype=np.int64)
            u[b] = ((j.astype(np.float64) + 0.5) / float(1 << 24)).astype(np.float32)
        else:
            raise RuntimeError(f"could not place uniforms of sequence {b} {eps} from thresholds")
    return u
