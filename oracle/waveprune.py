"""CPU oracle for WavePrune attention (RoPE first-period truncation).

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module.  The library
(rope_positional_encoding_amd, libwaveprune) never calls it, and it shares no
code with the library: it is numpy in float64, written from the pages'
definitions, slow and plain on purpose.

Sources (pages on "WavePrune: One period is often enough for RoPE",
arXiv 2610.06963):
  [notes]   cc.laoqi.cc reading notes "WavePrune：RoPE 通常只需一个旋转周期"
  [article] kongchang.com article "WavePrune：RoPE只用一个旋转周期，长文本性能反而更好"
  [thread]  the first author's thread on sotwe.com (tweets 3/7 and 6/7)

Readings taken where the pages leave a step open:
  * channel c is the interleaved pair of dims (2c, 2c+1) ([article], RoPE
    paragraph: the pair (q_{2i}, q_{2i+1}));
  * the 2x2 rotation is [[cos, -sin], [sin, cos]] applied to (x, y);
  * integer distances keep a channel iff dist <= floor(w_c) ([notes] §2.1);
  * linear position scaling s divides every frequency by s, for the rotation
    and for the cutoffs ([notes] §1.1: cutoffs come from the scaled
    frequencies);
  * grouped rule: group g is the dims [gG, (g+1)G) and its cutoff is the
    largest per-dim cutoff inside it ([notes] §2.3, Eq. (8));
  * GQA: query head h reads kv head h // (Hq/Hkv).

Parity status of every function: pinned (see tests/test_oracle_*.py).
"""
from __future__ import annotations

import math

import numpy as np

INT32_MAX = 2 ** 31 - 1
NEVER = INT32_MAX   # a cutoff that no distance exceeds: the channel is never pruned


# ----------------------------------------------------------------------------
# frequency schedule and cutoffs
# ----------------------------------------------------------------------------
def frequencies(theta: float, d_h: int, pos_scale: float = 1.0) -> np.ndarray:
    """f_c = theta^(-2c/d_h) radians per token, c = 0 .. d_h/2-1, divided by
    the linear position scale.  [notes] §1.1, frequency schedule (Eq. 2-5)."""
    c = np.arange(d_h // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * c / d_h) / float(pos_scale)


def wavelengths(theta: float, d_h: int, pos_scale: float = 1.0) -> np.ndarray:
    """w_c = 2*pi / f_c, in tokens.  [notes] §1.1."""
    return 2.0 * math.pi / frequencies(theta, d_h, pos_scale)


def channel_cutoffs(theta: float, d_h: int, pos_scale: float = 1.0) -> np.ndarray:
    """Largest kept integer distance per channel: floor(w_c), clamped to
    INT32_MAX.  [notes] §2.1, the note on integer distances after Eq. (6)."""
    w = np.floor(wavelengths(theta, d_h, pos_scale))
    return np.minimum(w, float(INT32_MAX)).astype(np.int64)


def group_cutoffs(theta: float, d_h: int, G: int, pos_scale: float = 1.0) -> np.ndarray:
    """d'_g = max over the scalar dims k of group g of d_k, where a dim
    inherits its channel's cutoff.  [notes] §2.3, Eq. (8)."""
    if G % 2 or d_h % G:
        raise ValueError("G must be even and divide d_h")
    per_dim = np.repeat(channel_cutoffs(theta, d_h, pos_scale), 2)
    return per_dim.reshape(d_h // G, G).max(axis=1)


def cutoffs_from_freqs(freqs, alpha: float = 2.0, trunc_channels=None) -> np.ndarray:
    """Per-channel cutoffs from an arbitrary per-channel frequency vector
    (radians per token, as the model rotates: any per-channel scaling
    already applied).  The window is w_c = alpha * pi / f_c: alpha = 2 is one
    period and alpha -> infinity prunes nothing; the kept integer distances
    are those <= floor(w_c) ([notes] §2.1, the paragraph after Eq. (6) on
    the pruning-strength knob alpha; §1.1 for cutoffs taken from the scaled
    frequencies).  Only channels c < trunc_channels are truncated ("only the
    first high-frequency channels", [notes] Appendix E summary and the
    Fig. 8a ablation axes); the rest are never pruned.  Values clamp to
    INT32_MAX."""
    f = np.asarray(freqs, dtype=np.float64)
    n_ch = f.shape[0]
    if trunc_channels is None:
        trunc_channels = n_ch
    out = np.full(n_ch, INT32_MAX, dtype=np.int64)
    if np.isinf(alpha):
        return out
    for c in range(min(trunc_channels, n_ch)):
        w = alpha * np.pi / f[c]
        out[c] = int(min(np.floor(w), float(INT32_MAX)))
    return out


def group_max(channel_cut: np.ndarray, G: int) -> np.ndarray:
    """Group table from per-channel cutoffs: every dim inherits its channel's
    cutoff and a group of G consecutive dims takes the largest
    ([notes] §2.3, Eq. (8))."""
    per_dim = np.repeat(np.asarray(channel_cut, dtype=np.int64), 2)
    d_h = per_dim.shape[0]
    if G % 2 or d_h % G:
        raise ValueError("G must be even and divide d_h")
    return per_dim.reshape(d_h // G, G).max(axis=1)


def dim_cutoffs_exact(theta: float, d_h: int, pos_scale: float = 1.0) -> np.ndarray:
    """Per-dim cutoff of the exact per-channel rule (Eq. 6)."""
    return np.repeat(channel_cutoffs(theta, d_h, pos_scale), 2)


def dim_cutoffs_grouped(group_cut: np.ndarray, G: int) -> np.ndarray:
    """Per-dim cutoff of the grouped rule: every dim of group g uses d'_g."""
    return np.repeat(np.asarray(group_cut, dtype=np.int64), G)


def dim_cutoffs_dense(d_h: int) -> np.ndarray:
    """Plain RoPE attention: nothing is ever pruned."""
    return np.full(d_h, NEVER, dtype=np.int64)


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------
def rope(x: np.ndarray, positions: np.ndarray, theta: float,
         pos_scale: float = 1.0) -> np.ndarray:
    """Rotate every channel of x [n, H, d_h] at token t by positions[t]*f_c.

    Channel c is the pair (x[2c], x[2c+1]) -> (x cos a - y sin a,
    x sin a + y cos a), a = p * f_c.  [notes] §1.1; [article] rotation matrix.
    """
    x = np.asarray(x, dtype=np.float64)
    d_h = x.shape[-1]
    f = frequencies(theta, d_h, pos_scale)
    a = np.asarray(positions, dtype=np.float64)[:, None] * f[None, :]   # [n, d_h/2]
    cos = np.cos(a)[:, None, :]
    sin = np.sin(a)[:, None, :]
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


# ----------------------------------------------------------------------------
# attention under a per-dim cutoff
# ----------------------------------------------------------------------------
def logits(q: np.ndarray, k: np.ndarray, dist: np.ndarray, dim_cut: np.ndarray) -> np.ndarray:
    """WavePrune logits of one query row against a set of keys.

    q [r, d_h] (the query heads that share one kv head), k [L, d_h] rotated
    keys, dist [L] = query position - key position (>= 0).  Each dim's
    product q[d]*k[d] counts only where dist <= dim_cut[d]; a truncated term
    is 0, not -inf, and the scale stays 1/sqrt(d_h).  [notes] §2.1, Eq. (6)
    and the three details after it; [thread] 3/7.
    Returns [r, L].
    """
    d_h = q.shape[-1]
    keep = (np.asarray(dist, dtype=np.int64)[:, None]
            <= np.asarray(dim_cut, dtype=np.int64)[None, :])          # [L, d_h]
    k_kept = np.asarray(k, dtype=np.float64) * keep                   # indicator per term
    return (np.asarray(q, dtype=np.float64) @ k_kept.T) / math.sqrt(d_h)


def softmax_av(L: np.ndarray, v: np.ndarray):
    """Row softmax over the (causal) keys, then A @ V; also the natural-log
    LSE.  [notes] §2.1, the softmax and Y = AV after Eq. (6)."""
    m = L.max(axis=1, keepdims=True)
    p = np.exp(L - m)
    s = p.sum(axis=1, keepdims=True)
    out = (p @ np.asarray(v, dtype=np.float64)) / s
    lse = (m + np.log(s))[:, 0]
    return out, lse


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, dim_cut: np.ndarray,
            rows=None, positions=None, return_lse: bool = False, q_is_rows: bool = False):
    """Causal WavePrune attention for one sequence.

    q [n, Hq, d_h], k/v [n, Hkv, d_h] (q and k already rotated); query row i
    sees keys j <= i; dist = positions[i] - positions[j] (default positions
    0..n-1, so dist = i - j).  With q_is_rows, q holds only the listed rows,
    in order.  Returns O [len(rows), Hq, d_h] (and LSE [len(rows), Hq]).
    """
    n = k.shape[0]
    Hq, d_h = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    r = Hq // Hkv
    pos = np.arange(n, dtype=np.int64) if positions is None else np.asarray(positions, np.int64)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), Hq, d_h), dtype=np.float64)
    lse = np.zeros((len(rows), Hq), dtype=np.float64)
    for idx, i in enumerate(rows):
        dist = pos[i] - pos[: i + 1]
        for kv in range(Hkv):
            hs = slice(kv * r, (kv + 1) * r)
            L = logits(q[idx if q_is_rows else i, hs, :], k[: i + 1, kv, :], dist, dim_cut)
            out[idx, hs], lse[idx, hs] = softmax_av(L, v[: i + 1, kv, :])
    return (out, lse) if return_lse else out


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, q_pos: int,
           cache_len: int, dim_cut: np.ndarray) -> np.ndarray:
    """One new query token at position q_pos against cached keys at positions
    0..cache_len-1 (all of them causal: q_pos >= cache_len - 1).

    q [Hq, d_h] rotated; k_cache/v_cache [>=cache_len, Hkv, d_h].
    Returns O [Hq, d_h].
    """
    if q_pos < cache_len - 1:
        raise ValueError("decode needs q_pos >= cache_len - 1")
    Hq, d_h = q.shape
    Hkv = k_cache.shape[1]
    r = Hq // Hkv
    dist = q_pos - np.arange(cache_len, dtype=np.int64)
    out = np.zeros((Hq, d_h), dtype=np.float64)
    for kv in range(Hkv):
        hs = slice(kv * r, (kv + 1) * r)
        L = logits(q[hs, :], k_cache[:cache_len, kv, :], dist, dim_cut)
        out[hs], _ = softmax_av(L, v_cache[:cache_len, kv, :])
    return out


def prefill_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, dim_cut: np.ndarray):
    """Gradients of the scalar <dO, O> with respect to q, k and v for the
    causal WavePrune attention of one sequence (the backward pass that the
    reading notes' section 2.3 describes for the kernel: the head dimension
    becomes an output axis, the gradient operands are masked per group, and
    dQ and dK share one mask).

    q [n, Hq, d_h], k/v [n, Hkv, d_h] (q, k rotated), do [n, Hq, d_h].
    Plain chain rule through O = softmax(S) V with
    S_ij = (1/sqrt(d_h)) sum_d keep(i-j, d) q_id k_jd, keep(t, d) = [t <= dim_cut[d]]:
      dV_j  = sum_i P_ij dO_i
      dP_ij = dO_i . V_j
      dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')        (softmax Jacobian)
      dQ_id = (1/sqrt(d_h)) sum_j dS_ij keep(i-j, d) k_jd
      dK_jd = (1/sqrt(d_h)) sum_i dS_ij keep(i-j, d) q_id
    summed over the query heads that share a kv head for dK and dV.  The dims
    are taken in classes of equal cutoff, each with one n x n mask.
    Returns dq [n, Hq, d_h], dk [n, Hkv, d_h], dv [n, Hkv, d_h] (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, Hq, d_h = q.shape
    Hkv = k.shape[1]
    r = Hq // Hkv
    sc = 1.0 / math.sqrt(d_h)
    cut = np.asarray(dim_cut, dtype=np.int64)
    dist = np.arange(n)[:, None] - np.arange(n)[None, :]          # i - j
    causal = dist >= 0
    classes = [(c, np.nonzero(cut == c)[0]) for c in np.unique(cut)]
    masks = [(dist <= c) & causal for c, _ in classes]
    dq = np.zeros_like(q)
    dk = np.zeros((n, Hkv, d_h))
    dv = np.zeros((n, Hkv, d_h))
    for h in range(Hq):
        kv = h // r
        S = np.zeros((n, n))
        for (c, dims), m in zip(classes, masks):
            S += (q[:, h, dims] @ k[:, kv, dims].T) * m
        S *= sc
        S = np.where(causal, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dv[:, kv] += P.T @ do[:, h]
        dP = do[:, h] @ v[:, kv].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        for (c, dims), m in zip(classes, masks):
            dSm = dS * m
            dq[:, h, dims] += sc * (dSm @ k[:, kv, dims])
            dk[:, kv, dims] += sc * (dSm.T @ q[:, h, dims])
    return dq, dk, dv


def prefill_backward_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                          dim_cut: np.ndarray, rows, key_from: int):
    """The backward pass of prefill_backward for sizes where the n x n
    matrices do not fit, restricted to a sample: dQ at the query rows `rows`,
    and what those rows contribute to dK and dV of the keys j >= key_from.

    Row by row, the same chain rule: with L_i the row's logits (logits()
    above), P_i = softmax(L_i), dP_ij = dO_i . V_j and
    dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij'):
      dQ_id = (1/sqrt(d_h)) sum_{j <= i} dS_ij keep(i-j, d) k_jd
      dK_jd += (1/sqrt(d_h)) dS_ij keep(i-j, d) q_id,   dV_j += P_ij dO_i.
    A key only receives gradient from rows at or after it (causality), so
    when `rows` holds every row >= key_from, the dK and dV returned are the
    complete gradients of the keys j >= key_from.
    Returns dq [len(rows), Hq, d_h], dk and dv [n - key_from, Hkv, d_h]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, Hq, d_h = q.shape
    Hkv = k.shape[1]
    r = Hq // Hkv
    sc = 1.0 / math.sqrt(d_h)
    cut = np.asarray(dim_cut, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((len(rows), Hq, d_h))
    dk = np.zeros((n - key_from, Hkv, d_h))
    dv = np.zeros((n - key_from, Hkv, d_h))
    for idx, i in enumerate(rows):
        dist = i - np.arange(i + 1)
        keep = dist[:, None] <= cut[None, :]                           # [i+1, d_h]
        for kv in range(Hkv):
            hs = slice(kv * r, (kv + 1) * r)
            L = logits(q[i, hs, :], k[: i + 1, kv, :], dist, cut)      # [r, i+1]
            P = np.exp(L - L.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dP = do[i, hs, :] @ v[: i + 1, kv, :].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[idx, hs, :] = sc * (dS @ (k[: i + 1, kv, :] * keep))
            if i >= key_from:
                js = slice(key_from, i + 1)
                dv[: i + 1 - key_from, kv, :] += P[:, js].T @ do[i, hs, :]
                dk[: i + 1 - key_from, kv, :] += sc * (dS[:, js].T @ q[i, hs, :]) * keep[js]
    return dq, dk, dv


# ----------------------------------------------------------------------------
# tile classification
# ----------------------------------------------------------------------------
SKIP, PARTIAL, FULL = 0, 1, 2


def classify(l_D: int, r_D: int, group_cut: np.ndarray) -> np.ndarray:
    """Per-group class of a tile whose causal distances span [l_D, r_D].
    [notes] §2.3 table: d'_g < l_D -> skip; l_D <= d'_g < r_D -> compute then
    mask; d'_g >= r_D -> full (no mask).  [thread] 6/7."""
    g = np.asarray(group_cut, dtype=np.int64)
    return np.where(g < l_D, SKIP, np.where(g < r_D, PARTIAL, FULL))


def classify_bruteforce(q_positions, k_positions, group_cut) -> np.ndarray:
    """Same classes from the pages' wording alone, by enumerating every causal
    pair of the tile: skip iff no pair is within the cutoff, full iff every
    pair is.  Returns None when the tile holds no causal pair."""
    qp = np.asarray(q_positions, dtype=np.int64)
    kp = np.asarray(k_positions, dtype=np.int64)
    d = (qp[:, None] - kp[None, :]).ravel()
    d = d[d >= 0]
    if d.size == 0:
        return None
    out = []
    for D in np.asarray(group_cut, dtype=np.int64):
        within = d <= D
        out.append(SKIP if not within.any() else FULL if within.all() else PARTIAL)
    return np.array(out)


def prefill_tile_counts(n: int, BM: int, BN: int, group_cut: np.ndarray):
    """Class counts over every visited (query block, key block) tile of one
    (sequence, query head): returns (counts [ng, 3] indexed by class, visited).
    A tile is visited when it holds a causal pair; tiles at the end are
    clipped to n.  Distances: l_D = max(0, i0 - j1), r_D = i1 - j0."""
    g = np.asarray(group_cut, dtype=np.int64)
    counts = np.zeros((len(g), 3), dtype=np.int64)
    visited = 0
    for i0 in range(0, n, BM):
        i1 = min(n, i0 + BM) - 1
        j0 = np.arange(0, i1 + 1, BN, dtype=np.int64)     # key blocks with j0 <= i1
        j1 = np.minimum(n, j0 + BN) - 1
        l_D = np.maximum(0, i0 - j1)
        r_D = i1 - j0
        visited += len(j0)
        for gi, D in enumerate(g):
            cls = np.where(D < l_D, SKIP, np.where(D < r_D, PARTIAL, FULL))
            counts[gi] += np.bincount(cls, minlength=3)
    return counts, visited


def decode_tile_counts(q_pos: int, cache_len: int, BN: int, group_cut: np.ndarray):
    """Class counts over the key blocks [j0, min(j0+BN, cache_len)-1] of one
    (sequence, kv head) in decode: l_D = q_pos - j1, r_D = q_pos - j0."""
    g = np.asarray(group_cut, dtype=np.int64)
    j0 = np.arange(0, cache_len, BN, dtype=np.int64)
    j1 = np.minimum(cache_len, j0 + BN) - 1
    l_D = q_pos - j1
    r_D = q_pos - j0
    counts = np.zeros((len(g), 3), dtype=np.int64)
    for gi, D in enumerate(g):
        cls = np.where(D < l_D, SKIP, np.where(D < r_D, PARTIAL, FULL))
        counts[gi] = np.bincount(cls, minlength=3)
    return counts, len(j0)
