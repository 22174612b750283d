"""Oracle: speculative-decoding verification, sequential and in float64 (test infrastructure).

What is computed, per sequence, following the modified rejection sampling algorithm
[P4 §"3. Mathematical Proof: Exact Distributional Match", §"The Modified Rejection Sampling
Algorithm"; P1 §"The core idea" (speculative_step); P3 §"Speculative Decoding: Turning
Verification Parallelism into Latency Wins" (speculative_generate)]:

* For draft position i = 0, 1, ..., k-1 in order, with draft token x_i, target probability
  p_i(x_i), draft probability q_i(x_i) and a uniform r_i: accept x_i when
  r_i <= min(1, p_i(x_i) / q_i(x_i)); otherwise reject it and stop checking.
* On the first rejection at position n, the replacement token is drawn from the residual
  max(0, p_n - q_n) normalised by its sum.
* If all k drafts are accepted, one bonus token is drawn from the target's row k.

Readings taken where the pages are silent or garbled:
* the test uses ``<=`` as in the formal statement (the pseudo-code listings use ``<``);
  uniforms lie in the open interval (0, 1);
* r <= min(1, P/Q) is evaluated exactly as ``P > 0 and r*Q <= P`` (a product of two fp32
  values is exact in fp64): Q = 0 < P accepts (ratio +inf), P = 0 always rejects;
* a draft id outside [0, V) has P = Q = 0 and is rejected;
* each sequence brings k+1 uniforms: r_0 .. r_{k-1} for the tests, u_k for the final draw;
* "sample from w" is the inverse CDF in ascending token id: t = u_k * Z with Z = sum(w) and
  C_x = w_0 + ... + w_x accumulated left to right in fp64; the token is the smallest x with
  C_x > t (strict, so a zero-weight token is never drawn);
* if Z == 0 (impossible for normalised rows after a rejection) the row p_n itself is used;
  if that is all zero too, token 0 is emitted; if rounding leaves no C_x > t, the largest x
  with w_x > 0 is taken;
* probabilities are used as given (no renormalisation beyond Z).
"""

from __future__ import annotations

import numpy as np


def sample_inverse_cdf(w: np.ndarray, u: float) -> int:
    """Smallest x with C_x > u * Z, C = running fp64 sum of w in ascending id (Z = C[-1])."""
    w = np.asarray(w, dtype=np.float64)
    total = 0.0
    cum = np.empty_like(w)
    for x in range(w.size):          # left-to-right accumulation, written out on purpose
        total += w[x]
        cum[x] = total
    Z = total
    if not Z > 0.0:
        return -1
    t = float(np.float64(u) * Z)
    above = np.nonzero(cum > t)[0]
    if above.size:
        return int(above[0])
    return int(np.nonzero(w > 0.0)[0][-1])


def accept_draft(P: float, Qx: float, r: float) -> bool:
    """r <= min(1, P/Qx), decided exactly: P > 0 and r*Qx <= P."""
    return bool(P > 0.0 and np.float64(r) * np.float64(Qx) <= np.float64(P))


def verify_sequence(p_rows: np.ndarray, q_rows: np.ndarray, drafts, uniforms):
    """One sequence.  p_rows [k+1, V], q_rows [k, V], drafts [k], uniforms [k+1].

    Returns (out_ids [k+1] with -1 after the emitted tokens, n_accepted).
    """
    p_rows = np.asarray(p_rows, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = len(drafts)
    V = p_rows.shape[1]
    out = np.full(k + 1, -1, dtype=np.int64)
    n = k
    for i in range(k):
        x = int(drafts[i])
        inside = 0 <= x < V
        P = p_rows[i, x] if inside else 0.0
        Qx = q_rows[i, x] if inside else 0.0
        if accept_draft(P, Qx, uniforms[i]):
            out[i] = x
        else:
            n = i
            break
    if n < k:
        w = np.maximum(0.0, p_rows[n] - q_rows[n])   # residual max(0, p - q)
    else:
        w = p_rows[k]                                 # bonus row
    y = sample_inverse_cdf(w, uniforms[k])
    if y < 0:                                         # Z == 0: fall back to p_n itself
        y = sample_inverse_cdf(p_rows[n], uniforms[k])
        if y < 0:
            y = 0
    out[n] = y
    return out, n


def spec_verify(p: np.ndarray, q: np.ndarray, draft_ids: np.ndarray, uniforms: np.ndarray):
    """Batch wrapper: p [B, k+1, V], q [B, k, V], draft_ids [B, k], uniforms [B, k+1].

    Returns (out_ids [B, k+1] int64, n_accepted [B] int64).
    """
    B = p.shape[0]
    k = q.shape[1]
    out = np.empty((B, k + 1), dtype=np.int64)
    n_acc = np.empty(B, dtype=np.int64)
    for b in range(B):
        out[b], n_acc[b] = verify_sequence(p[b], q[b], draft_ids[b], uniforms[b])
    return out, n_acc


# ----------------------------------------------------------------------------------------
# decision margins: used by the test harness to draw uniforms that sit at least eps away
# from every threshold the algorithm actually evaluates, so that summation order cannot
# change a decision between two correct implementations.
# ----------------------------------------------------------------------------------------

def decision_margin(p_rows, q_rows, drafts, uniforms) -> float:
    """Smallest |u - threshold| over the decisions the oracle takes for one sequence.

    Accept tests: |r_i - min(1, P/Q)| for i up to the first rejection.
    Final draw:   |u_k - C_x / Z| for every x of the row that is sampled.
    """
    p_rows = np.asarray(p_rows, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = len(drafts)
    V = p_rows.shape[1]
    margin = np.inf
    n = k
    for i in range(k):
        x = int(drafts[i])
        inside = 0 <= x < V
        P = p_rows[i, x] if inside else 0.0
        Qx = q_rows[i, x] if inside else 0.0
        if Qx > 0.0:
            margin = min(margin, abs(float(uniforms[i]) - min(1.0, P / Qx)))
        if not accept_draft(P, Qx, uniforms[i]):
            n = i
            break
    w = np.maximum(0.0, p_rows[n] - q_rows[n]) if n < k else p_rows[k]
    if not w.sum() > 0.0:
        w = p_rows[n]
    cum = np.cumsum(w)
    if cum[-1] > 0.0:
        margin = min(margin, float(np.min(np.abs(float(uniforms[k]) - cum / cum[-1]))))
    return margin


def uniforms_with_margin(p, q, draft_ids, uniforms, rng: np.random.Generator, eps: float = 1e-6,
                         max_tries: int = 1000) -> np.ndarray:
    """Redraw (seeded) every sequence's uniforms until its decision margin is >= eps."""
    u = np.array(uniforms, dtype=np.float32, copy=True)
    for b in range(p.shape[0]):
        for _ in range(max_tries):
            if decision_margin(p[b], q[b], draft_ids[b], u[b]) >= eps:
                break
            j = rng.integers(0, 1 << 24, size=u.shape[1], dtype=np.int64)
            u[b] = ((j.astype(np.float64) + 0.5) / float(1 << 24)).astype(np.float32)
        else:
            raise RuntimeError(f"could not place uniforms of sequence {b} {eps} from thresholds")
    return u
