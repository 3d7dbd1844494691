"""Pins for the oracle's attention (exact rule, grouped rule, decode).

* With every cutoff infinite the method is plain causal RoPE attention, so the
  oracle must agree with torch's CPU scaled_dot_product_attention in float64.
* A scalar brute force (explicit 2x2 rotation matrices, one channel at a time,
  the indicator tested per channel) on tiny inputs, with a small theta so that
  pruned, partially pruned and fully pruned key rows all occur.
* Invariants: G = 2 grouped == exact; grouped keep-set contains the exact one;
  a common position shift changes nothing; decode == the prefill row.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _bruteforce(q_raw, k_raw, v, pos, theta, chan_cut):
    """Scalar loops: rotate each channel by its own 2x2 matrix, add a channel's
    dot product only when the distance is within its cutoff (a pruned channel
    adds 0), softmax over j <= i, weighted sum of V."""
    n, Hq, d = q_raw.shape
    Hkv = k_raw.shape[1]
    out = np.zeros((n, Hq, d))
    for i in range(n):
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            lg = []
            for j in range(i + 1):
                dist = pos[i] - pos[j]
                acc = 0.0
                for c in range(d // 2):
                    f = theta ** (-2.0 * c / d)
                    Ri = np.array([[math.cos(pos[i] * f), -math.sin(pos[i] * f)],
                                   [math.sin(pos[i] * f), math.cos(pos[i] * f)]])
                    Rj = np.array([[math.cos(pos[j] * f), -math.sin(pos[j] * f)],
                                   [math.sin(pos[j] * f), math.cos(pos[j] * f)]])
                    qc = Ri @ q_raw[i, h, 2 * c:2 * c + 2]
                    kc = Rj @ k_raw[j, kv, 2 * c:2 * c + 2]
                    if dist <= chan_cut[c]:
                        acc += float(qc @ kc)
                lg.append(acc / math.sqrt(d))
            lg = np.array(lg)
            w = np.exp(lg - lg.max())
            w /= w.sum()
            out[i, h] = w @ v[: i + 1, kv]
    return out


def _inputs(seed, n, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, Hq, d)), rng.standard_normal((n, Hkv, d)),
            rng.standard_normal((n, Hkv, d)))


@pytest.mark.parametrize("theta,d,G,n,p0", [(100.0, 8, 4, 40, 0), (30.0, 8, 8, 33, 5),
                                             (1e4, 16, 16, 24, 3), (4.0, 4, 4, 30, 2)])
def test_bruteforce_exact_and_grouped(theta, d, G, n, p0):
    q, k, v = _inputs(11, n, 2, 1, d)
    pos = np.arange(n) + p0
    qr = O.rope(q, pos, theta)
    kr = O.rope(k, pos, theta)
    # exact rule: per-channel cutoffs
    ch = O.channel_cutoffs(theta, d)
    got = O.prefill(qr, kr, v, O.dim_cutoffs_exact(theta, d), positions=pos)
    assert np.allclose(got, _bruteforce(q, k, v, pos, theta, ch), atol=1e-12)
    # grouped rule: every channel of group g uses the group's max
    g = O.group_cutoffs(theta, d, G)
    ch_g = np.repeat(g, G // 2)
    got_g = O.prefill(qr, kr, v, O.dim_cutoffs_grouped(g, G), positions=pos)
    assert np.allclose(got_g, _bruteforce(q, k, v, pos, theta, ch_g), atol=1e-12)


def test_fully_pruned_keys_keep_logit_zero():
    # theta = 100, d_h = 8: every channel is pruned beyond distance 198; those
    # keys get logit exactly 0 and still take softmax mass (not -inf).
    theta, d, n = 100.0, 8, 260
    q, k, v = _inputs(12, n, 1, 1, d)
    pos = np.arange(n)
    qr, kr = O.rope(q, pos, theta), O.rope(k, pos, theta)
    cut = O.dim_cutoffs_exact(theta, d)
    i = n - 1
    L = O.logits(qr[i], kr[: i + 1, 0], i - pos[: i + 1], cut)[0]
    far = (i - pos[: i + 1]) > 198
    assert far.sum() == i + 1 - 199
    assert np.all(L[far] == 0.0)
    # with V = indicator of the far keys, O = (#far) / (sum_near e^L + #far)
    ind = far.astype(np.float64)[:, None] * np.ones((1, d))
    vv = np.zeros((n, 1, d))
    vv[: i + 1, 0] = ind
    out = O.prefill(qr, kr, vv, cut, rows=[i])[0, 0, 0]
    expect = far.sum() / (np.exp(L[~far]).sum() + far.sum())
    assert abs(out - expect) < 1e-12


@pytest.mark.parametrize("Hq,Hkv,d,n", [(4, 2, 16, 50), (8, 2, 32, 70), (1, 1, 64, 33)])
def test_infinite_cutoffs_is_sdpa(Hq, Hkv, d, n):
    q, k, v = _inputs(13, n, Hq, Hkv, d)
    pos = np.arange(n)
    qr, kr = O.rope(q, pos, 1e4), O.rope(k, pos, 1e4)
    got, lse = O.prefill(qr, kr, v, O.dim_cutoffs_dense(d), return_lse=True)
    r = Hq // Hkv
    tq = torch.from_numpy(qr).permute(1, 0, 2)[None]
    tk = torch.from_numpy(kr).permute(1, 0, 2).repeat_interleave(r, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(r, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.allclose(got, ref, atol=1e-12)
    # LSE against torch.logsumexp of the masked score matrix
    s = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1)[0].permute(1, 0).numpy()
    assert np.allclose(lse, ref_lse, atol=1e-12)


def test_grouped_G2_equals_exact():
    q, k, v = _inputs(14, 90, 4, 2, 32)
    pos = np.arange(90)
    qr, kr = O.rope(q, pos, 50.0), O.rope(k, pos, 50.0)
    a = O.prefill(qr, kr, v, O.dim_cutoffs_exact(50.0, 32))
    b = O.prefill(qr, kr, v, O.dim_cutoffs_grouped(O.group_cutoffs(50.0, 32, 2), 2))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("p0", [1000, 12345])
def test_common_shift_changes_nothing(p0):
    theta, d, n = 1e4, 32, 120
    q, k, v = _inputs(15, n, 2, 1, d)
    cut = O.dim_cutoffs_grouped(O.group_cutoffs(theta, d, 8), 8)
    base = O.prefill(O.rope(q, np.arange(n), theta), O.rope(k, np.arange(n), theta), v, cut)
    pos = np.arange(n) + p0
    sh = O.prefill(O.rope(q, pos, theta), O.rope(k, pos, theta), v, cut, positions=pos)
    assert np.allclose(base, sh, atol=1e-12)


def test_kept_pair_count_closed_form():
    # one dim with cutoff D: the causal pairs (i, j) of an n x n map with
    # i - j <= D number (D + 1)(2n - D)/2 for D < n.
    n, d = 64, 4
    for D in (0, 1, 7, 30, 63):
        cut = np.array([D, O.NEVER, O.NEVER, O.NEVER])
        q = np.zeros((1, d))
        q[0, 0] = 1.0
        k = np.zeros((n, d))
        k[:, 0] = 1.0
        kept = 0
        for i in range(n):
            L = O.logits(q, k[: i + 1], i - np.arange(i + 1), cut)
            kept += int((L != 0).sum())
        assert kept == (D + 1) * (2 * n - D) // 2


def test_rows_are_convex_combinations():
    q, k, v = _inputs(16, 40, 2, 2, 16)
    pos = np.arange(40)
    cut = O.dim_cutoffs_exact(30.0, 16)
    ones = np.ones_like(v)
    out = O.prefill(O.rope(q, pos, 30.0), O.rope(k, pos, 30.0), ones, cut)
    assert np.allclose(out, 1.0, atol=1e-14)
    # row 0 sees only key 0
    out = O.prefill(O.rope(q, pos, 30.0), O.rope(k, pos, 30.0), v, cut, rows=[0])
    assert np.allclose(out[0], v[0][[0, 1]], atol=1e-14)


def test_decode_equals_prefill_row():
    theta, d, n = 1e3, 32, 150
    q, k, v = _inputs(17, n, 4, 2, d)
    pos = np.arange(n)
    qr, kr = O.rope(q, pos, theta), O.rope(k, pos, theta)
    cut = O.dim_cutoffs_grouped(O.group_cutoffs(theta, d, 16), 16)
    for i in (0, 1, 77, n - 1):
        pre = O.prefill(qr, kr, v, cut, rows=[i])[0]
        dec = O.decode(qr[i], kr, v, q_pos=i, cache_len=i + 1, dim_cut=cut)
        assert np.allclose(pre, dec, atol=1e-13)
    # a query one past the cache (its own K/V not cached): distances 1..L
    L = 100
    dec = O.decode(qr[L], kr, v, q_pos=L, cache_len=L, dim_cut=cut)
    lg = np.stack([O.logits(qr[L, h:h + 1], kr[:L, h // 2], L - np.arange(L), cut)[0]
                   for h in range(4)])
    w = np.exp(lg - lg.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    ref = np.stack([w[h] @ v[:L, h // 2] for h in range(4)])
    assert np.allclose(dec, ref, atol=1e-13)
