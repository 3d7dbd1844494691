"""Element-wise error bound for the GPU backward gradients (test helper, not
collected: no test_ prefix).

The GPU backward takes bf16 q, k, v, dO (exact inputs), the forward's bf16 O
and float32 LSE, recomputes P in float32, rounds P (for dV += P^T dO) and
dS = P (dP - D) (for dK and dQ) to bf16 MFMA operands, accumulates in
float32 and rounds each gradient to bf16.  With u = 2^-8, the unit roundoff
of bf16 (8 significant bits, round to nearest even), every gradient element
is a float32 sum of terms a_t (1 + delta_t) with |delta_t| <= u, plus the
row term D_i = dO_i . O_i taken from the forward's O, whose own error is its
bf16 output rounding (<= u |O|) plus the sum of its rounded P terms.

Bound used by the tests, element by element:

    |gpu - oracle| <= u |oracle| + C u sqrt(R) + 1e-6

  * u |oracle|: the bf16 rounding of the output;
  * C u sqrt(R): the rounded operand terms.  The rounding errors of distinct
    terms are independent, zero-mean and bounded by u |a_t|, so by
    Hoeffding's inequality P(|sum_t a_t delta_t| > C u sqrt(sum_t a_t^2))
    <= 2 exp(-C^2 / 2); C = 8 makes that 2.5e-14 per element;
  * R sums the squared terms:
      dV_jd: a = P_ij dO_id                                 (bf16 P)
      dK_jd: a = s keep_ijd (|dS_ij| + P_ij E_i) q_id        (bf16 dS, D from O)
      dQ_id: a = s keep_ijd (|dS_ij| + P_ij E_i) k_jd
    with s = 1/sqrt(d_h) and E_i = C sqrt(sum_d dO_id^2 O_id^2) + C sqrt(sum_j P_ij^2 dP_ij^2),
    the bound on the error of D_i divided by u: the bf16 rounding of each O_id,
    and the forward's rounding of each P_ij, which enters D_i as
    sum_j P_ij delta_ij (dO_i . V_j) = sum_j P_ij delta_ij dP_ij;
  * 1e-6: float32 accumulation of at most 2^17 terms of size <= 1, far below
    the rest.
dK and dV also sum over the query heads of their kv head.

P, dP and dS are taken from the oracle's own logits (oracle.logits), so the
keep rule is the oracle's.
"""
from __future__ import annotations

import math

import numpy as np

import oracle as O

U = 2.0 ** -8
C = 8.0
FLOOR = 1e-6


def backward_terms(q, k, v, do, dim_cut, rows=None, key_from: int = 0):
    """Sum of squared rounded terms R for dQ at `rows` ([len(rows), Hq, d])
    and for dK, dV of the keys j >= key_from ([n - key_from, Hkv, d]),
    complete for those keys when `rows` holds every row >= key_from."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    r = Hq // Hkv
    s2 = 1.0 / d
    cut = np.asarray(dim_cut, dtype=np.int64)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    Rq = np.zeros((len(rows), Hq, d))
    Rk = np.zeros((n - key_from, Hkv, d))
    Rv = np.zeros((n - key_from, Hkv, d))
    for idx, i in enumerate(rows):
        dist = i - np.arange(i + 1)
        keep = (dist[:, None] <= cut[None, :]).astype(np.float64)      # [i+1, d]
        for kv in range(Hkv):
            hs = slice(kv * r, (kv + 1) * r)
            kk, vv = k[: i + 1, kv], v[: i + 1, kv]
            L = O.logits(q[i, hs], kk, dist, cut)                     # [r, i+1]
            P = np.exp(L - L.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            g = do[i, hs]                                              # [r, d]
            dP = g @ vv.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            o = P @ vv                                                 # exact O rows [r, d]
            E = C * np.sqrt(((g * o) ** 2).sum(axis=1)) + C * np.sqrt(((P * dP) ** 2).sum(axis=1))
            F2 = (np.abs(dS) + P * E[:, None]) ** 2                    # [r, i+1]
            Rq[idx, hs] = s2 * (F2 @ (kk ** 2 * keep))
            if i >= key_from:
                js = slice(key_from, i + 1)
                Rv[: i + 1 - key_from, kv] += (P[:, js] ** 2).T @ (g ** 2)
                Rk[: i + 1 - key_from, kv] += s2 * (F2[:, js].T @ (q[i, hs] ** 2)) * keep[js]
    return Rq, Rk, Rv


def check(got, ref, R, label, say=print):
    """Assert |got - ref| <= U |ref| + C U sqrt(R) + FLOOR element-wise, and
    report the worst ratio of error to bound."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    bound = U * np.abs(ref) + C * U * np.sqrt(R) + FLOOR
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    say("  %s: max-abs %.2e, mean-abs %.2e, max |ref| %.3g, worst err/bound %.3f (err %.2e, bound %.2e)"
        % (label, err.max(), err.mean(), np.abs(ref).max(), ratio[worst], err[worst], bound[worst]))
    assert np.all(np.isfinite(got)), label
    assert np.all(err <= bound), (label, float(ratio[worst]), worst)
    return float(ratio[worst])
