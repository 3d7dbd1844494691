"""Pins from the pages' analysis of periodicity (reading notes §1.1 and §2.2,
Theorem 1 and its proof sketch; thread 2/7 and 3/7).

With a constant query q and key k at every position, plain RoPE's logit
depends on the lag only: L(lag) = (1/sqrt(d_h)) sum_c |q_c||k_c| cos(lag f_c
+ w_c), a closed form independent of the oracle's code.  Theorem 1 says lags
far beyond the first period come back within tau of the supremum ("ghost
sub-diagonals"); after truncation every lag beyond the largest cutoff has
logit exactly 0, so none can.
"""
import math

import numpy as np

import oracle as O


def _const_logits(q, k, N, theta, cut):
    """Oracle logits of the last row of a length-N sequence with q_i = q and
    k_j = k for every position; returns L indexed by lag 0..N-1."""
    d = q.shape[-1]
    pos = np.arange(N)
    qr = O.rope(np.broadcast_to(q, (1, 1, d)).copy(), pos[-1:], theta)[0]   # [1, d]
    kr = O.rope(np.broadcast_to(k, (N, 1, d)).copy(), pos, theta)[:, 0]       # [N, d]
    L = O.logits(qr, kr, (N - 1) - pos, cut)[0]                              # by key
    return L[::-1]                                                           # by lag


def test_constant_qk_closed_form():
    rng = np.random.default_rng(21)
    d, theta, N = 16, 500.0, 700
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    L = _const_logits(q, k, N, theta, O.dim_cutoffs_dense(d))
    zq = q[0::2] + 1j * q[1::2]
    zk = k[0::2] + 1j * k[1::2]
    f = theta ** (-2.0 * np.arange(d // 2) / d)
    lag = np.arange(N)
    # channel term: |q_c||k_c| cos(lag f_c + w_c), w_c = arg q_c - arg k_c
    w = np.angle(zq) - np.angle(zk)
    ref = (np.abs(zq) * np.abs(zk) * np.cos(lag[:, None] * f + w)).sum(1) / math.sqrt(d)
    assert np.allclose(L, ref, atol=1e-10)


def test_ghost_subdiagonals_and_their_removal():
    # d_h = 8, theta = 100: cutoffs 6/19/62/198; N = 4000; tau = 0.1 L*
    rng = np.random.default_rng(22)
    d, theta, N = 8, 100.0, 4000
    q = rng.standard_normal(d)
    plain = _const_logits(q, q, N, theta, O.dim_cutoffs_dense(d))
    Lstar = plain.max()
    assert abs(Lstar - plain[0]) < 1e-12            # q = k: the peak is lag 0
    tau = 0.1 * Lstar
    ghosts = np.nonzero(plain[199:] >= Lstar - tau)[0] + 199
    assert len(ghosts) >= 5                        # lags far past every period
    wp = _const_logits(q, q, N, theta, O.dim_cutoffs_exact(theta, d))
    assert np.all(wp[199:] == 0.0)                 # truncated: exactly 0
    assert not np.any(wp[199:] >= Lstar - tau)
    assert np.allclose(wp[:7], plain[:7], atol=1e-12)   # nothing pruned at lag <= 6


def test_lipschitz_bound_on_shifts():
    # |L(lag+P) - L(lag)| <= (1/sqrt d) sum_c m_c^Q m_c^K |wrap(P f_c)|
    rng = np.random.default_rng(23)
    d, theta, N = 16, 1e3, 3000
    for _ in range(3):
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        L = _const_logits(q, k, N, theta, O.dim_cutoffs_dense(d))
        mq = np.hypot(q[0::2], q[1::2])
        mk = np.hypot(k[0::2], k[1::2])
        f = theta ** (-2.0 * np.arange(d // 2) / d)
        for P in rng.integers(1, 1500, size=20):
            wrap = np.abs((P * f + np.pi) % (2 * np.pi) - np.pi)
            bound = (mq * mk * wrap).sum() / math.sqrt(d)
            lag = np.arange(N - P)
            assert np.all(np.abs(L[lag + P] - L[lag]) <= bound + 1e-9)
