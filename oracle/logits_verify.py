"""Oracle: speculative verification that starts from logits (test infrastructure only).

What is computed, per sequence:

* The verify pass returns target logits, one row per draft position plus one
  [P3 §"Speculative Decoding: Turning Verification Parallelism into Latency Wins": the target's
  verify call yields logits of shape [gamma + 1, vocab], and sample(logits) draws a token from
  logits].  With a sampling temperature T > 0 the target and draft distributions are
      p_i = softmax(z_p,i / T),   q_i = softmax(z_q,i / T)      (fp64),
  and the modified rejection sampling rule of ``oracle.spec_verify`` runs on them
  [P4 §"The Modified Rejection Sampling Algorithm"].
* At temperature 0 speculative decoding reduces to exact token matching [P3 §"Frequently Asked
  Questions"; same page, "at temperature 0, speculative decoding is exact"].  T = 0 is read as
  the greedy limit: p_i and q_i are one-hot at their row's first argmax, and the same rule runs
  on them.  It accepts x_i exactly while x_i is the target row's argmax and emits the argmax of
  row n (the residual is then the target's one-hot, or empty and replaced by p_n).

Readings taken where the pages are silent:
* one temperature per sequence, shared by the target and the draft rows (the draft tokens were
  drawn with the same sampling setting);
* argmax ties go to the smallest token id;
* the softmax subtracts the row maximum before exponentiating (the value is the same; it only
  keeps exp finite for large logits).
"""

from __future__ import annotations

import numpy as np

from . import spec_verify as S


def tempered_softmax(z, T: float) -> np.ndarray:
    """softmax(z / T) over the last axis, in fp64."""
    y = np.asarray(z, dtype=np.float64) / float(T)
    y = y - y.max(axis=-1, keepdims=True)
    e = np.exp(y)
    return e / e.sum(axis=-1, keepdims=True)


def greedy_rows(z) -> np.ndarray:
    """One-hot rows at the first argmax of each row of z (the T -> 0 limit of the softmax)."""
    z = np.asarray(z)
    out = np.zeros(z.shape, dtype=np.float64)
    idx = np.argmax(z, axis=-1)
    np.put_along_axis(out, idx[..., None], 1.0, axis=-1)
    return out


def distributions(zp, zq, T: float):
    """(p [k+1, V], q [k, V]) of one sequence at temperature T."""
    if T == 0.0:
        return greedy_rows(zp), greedy_rows(zq)
    return tempered_softmax(zp, T), tempered_softmax(zq, T)


def verify_logits_sequence(zp, zq, drafts, uniforms, T: float):
    """One sequence: zp [k+1, V] target logits, zq [k, V] draft logits, drafts [k],
    uniforms [k+1], temperature T >= 0.  Returns (out_ids [k+1], n_accepted)."""
    if not (np.isfinite(T) and T >= 0.0):
        raise ValueError("temperature must be finite and >= 0")
    p, q = distributions(zp, zq, float(T))
    return S.verify_sequence(p, q, drafts, uniforms)


def verify_logits(zp: np.ndarray, zq: np.ndarray, draft_ids: np.ndarray, uniforms: np.ndarray, temps):
    """Batch wrapper: zp [B, k+1, V], zq [B, k, V], draft_ids [B, k], uniforms [B, k+1],
    temps [B].  Returns (out_ids [B, k+1] int64, n_accepted [B] int64)."""
    B, k1, _ = zp.shape
    out = np.empty((B, k1), dtype=np.int64)
    n_acc = np.empty(B, dtype=np.int64)
    for b in range(B):
        out[b], n_acc[b] = verify_logits_sequence(zp[b], zq[b], draft_ids[b], uniforms[b], float(temps[b]))
    return out, n_acc


def uniforms_with_margin(zp, zq, draft_ids, uniforms, temps, rng: np.random.Generator, eps: float = 1e-6):
    """Seeded redraw of each sequence's uniforms until every decision the oracle takes on it
    sits at least eps from its threshold (see ``oracle.spec_verify.decision_margin``)."""
    u = np.array(uniforms, dtype=np.float32, copy=True)
    for b in range(zp.shape[0]):
        p, q = distributions(zp[b], zq[b], float(temps[b]))
        u[b] = S.uniforms_with_margin(p[None], q[None], draft_ids[b][None], u[b][None], rng, eps)[0]
    return u
