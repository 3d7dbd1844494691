"""Pins for the oracle's frequency schedule, cutoffs and RoPE.

Each check compares the oracle with something other than itself: values the
pages print, hand-computed closed forms, or a different mathematical
formulation (complex multiplication).
"""
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


def test_table12_printed_wavelengths():
    # reading notes §4.7 (Table 12): last channel of each group, theta=1e6, d_h=128
    rows = _rows("table12_wavelengths.txt")
    w = O.wavelengths(1e6, 128)
    D = O.channel_cutoffs(1e6, 128)
    g16 = O.group_cutoffs(1e6, 128, 16)
    for gi, (ch, printed) in enumerate(rows):
        ch, printed = int(ch), int(printed)
        assert round(w[ch]) == printed or int(w[ch]) == printed
        assert D[ch] == printed          # floor of the printed-rounded value
        assert g16[gi] == printed        # group max = the group's last channel


def test_worked_example_section21():
    rows = _rows("worked_example_channels.txt")
    w = O.wavelengths(1e6, 128)
    D = O.channel_cutoffs(1e6, 128)
    for ch, printed, tol, kept in rows:
        ch = int(ch)
        assert abs(w[ch] - float(printed)) <= float(tol)
        # a single non-zero channel: its logit at distance 100 is non-zero iff kept
        q = np.zeros((1, 128))
        k = np.zeros((1, 128))
        q[0, 2 * ch] = 1.0
        k[0, 2 * ch] = 1.0
        L = O.logits(q, k, np.array([100]), O.dim_cutoffs_exact(1e6, 128))
        assert (L[0, 0] != 0) == bool(int(kept))
        assert (100 <= D[ch]) == bool(int(kept))


def test_cutoffs_hand_computed_small():
    # f_c = 100^(-2c/8): 1, 100^-0.25, 0.1, 100^-0.75 -> w = 2pi * (1, 3.1623, 10, 31.623)
    assert list(O.channel_cutoffs(100.0, 8)) == [6, 19, 62, 198]
    # theta = 1e4, d_h = 64, G = 16: group maxima are channels 7, 15, 23, 31
    # w = 2pi * 10^(c/8) at c = 7, 15, 23, 31 -> 47.12, 471.17, 4711.74, 47117.4
    assert list(O.group_cutoffs(1e4, 64, 16)) == [47, 471, 4711, 47117]


def test_linear_scale_multiplies_wavelength_before_floor():
    # position interpolation by s divides every frequency by s: w -> s*w
    w1 = O.wavelengths(1e6, 128)
    D4 = O.channel_cutoffs(1e6, 128, 4.0)
    assert np.array_equal(D4, np.floor(4.0 * w1).astype(np.int64))
    assert list(O.group_cutoffs(1e6, 128, 16, 4.0)[:3]) == [113, 640, 3601]


def test_group_rule_structure():
    for theta, d_h, s in [(1e4, 64, 1.0), (1e6, 128, 1.0), (1e6, 128, 4.0), (500.0, 32, 2.0)]:
        ex = O.dim_cutoffs_exact(theta, d_h, s)
        assert np.array_equal(O.group_cutoffs(theta, d_h, 2, s), O.channel_cutoffs(theta, d_h, s))
        for G in (2, 4, 8, 16, 32):
            if d_h % G:
                continue
            g = O.group_cutoffs(theta, d_h, G, s)
            assert np.all(np.diff(g) >= 0)                       # monotone
            gr = O.dim_cutoffs_grouped(g, G)
            assert np.all(gr >= ex)                               # keep-set superset
            assert np.array_equal(g, ex.reshape(-1, G)[:, -1])   # = last dim of group


def test_general_cutoffs_hand_computed():
    # w_c = alpha * pi / f_c, kept distances <= floor(w_c); by hand:
    # f = [1, 0.5, 0.25]: alpha 2 -> floor(2pi)=6, floor(4pi)=12, floor(8pi)=25
    f = [1.0, 0.5, 0.25]
    assert list(O.cutoffs_from_freqs(f, 2.0)) == [6, 12, 25]
    # alpha 1 (half a period): floor(pi)=3, floor(2pi)=6, floor(4pi)=12
    assert list(O.cutoffs_from_freqs(f, 1.0)) == [3, 6, 12]
    # alpha 3: floor(3pi)=9, floor(6pi)=18, floor(12pi)=37
    assert list(O.cutoffs_from_freqs(f, 3.0)) == [9, 18, 37]
    # only the first channel truncated; the others never pruned
    assert list(O.cutoffs_from_freqs(f, 2.0, trunc_channels=1)) == [6, O.INT32_MAX, O.INT32_MAX]
    # nothing truncated, and alpha -> infinity, both prune nothing
    assert all(v == O.INT32_MAX for v in O.cutoffs_from_freqs(f, 2.0, trunc_channels=0))
    assert all(v == O.INT32_MAX for v in O.cutoffs_from_freqs(f, math.inf))
    # a vanishing frequency clamps to the never-prune value
    assert O.cutoffs_from_freqs([1e-12], 2.0)[0] == O.INT32_MAX
    # group of two channels (G = 4) takes the larger: [6, 12] -> 12, [25] alone with G=2
    assert list(O.group_max([6, 12], 4)) == [12]
    assert list(O.group_max([6, 12, 25], 2)) == [6, 12, 25]


def test_general_cutoffs_reduce_to_theta_schedule():
    # with the plain schedule, alpha = 2 and every channel truncated, the
    # general table is the theta table (itself pinned to Table 12 above)
    for theta, d_h, s in [(1e4, 64, 1.0), (1e6, 128, 1.0), (1e6, 128, 4.0), (5e5, 128, 2.5)]:
        f = O.frequencies(theta, d_h, s)
        ch = O.cutoffs_from_freqs(f, 2.0)
        assert np.array_equal(ch, O.channel_cutoffs(theta, d_h, s))
        for G in (2, 16, 32):
            assert np.array_equal(O.group_max(ch, G), O.group_cutoffs(theta, d_h, G, s))


def test_general_cutoffs_monotone_in_alpha_and_truncation():
    f = O.frequencies(1e6, 128)
    prev = None
    for alpha in (0.5, 1.0, 1.9, 2.0, 2.5, 8.0):
        cur = O.cutoffs_from_freqs(f, alpha)
        if prev is not None:
            assert np.all(cur >= prev)
        prev = cur
    full = O.cutoffs_from_freqs(f, 2.0)
    for k in (0, 1, 17, 63, 64):
        part = O.cutoffs_from_freqs(f, 2.0, trunc_channels=k)
        assert np.array_equal(part[:k], full[:k])
        assert np.all(part[k:] == O.INT32_MAX)


def test_rope_hand_example():
    # d_h = 4, theta = 100: f = (1, 0.1); position 3; x = (1, 0, 0, 1)
    x = np.array([[[1.0, 0.0, 0.0, 1.0]]])
    y = O.rope(x, np.array([3]), 100.0)[0, 0]
    expect = [math.cos(3.0), math.sin(3.0), -math.sin(0.3), math.cos(0.3)]
    assert np.allclose(y, expect, atol=1e-15)


def test_rope_is_complex_multiplication():
    rng = np.random.default_rng(7)
    n, H, d = 37, 3, 32
    x = rng.standard_normal((n, H, d))
    pos = rng.integers(0, 200000, size=n)
    theta, s = 1e6, 4.0
    y = O.rope(x, pos, theta, s)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    c = np.arange(d // 2)
    ang = pos[:, None] * (theta ** (-2.0 * c / d) / s)
    zr = z * np.exp(1j * ang)[:, None, :]
    assert np.allclose(y[..., 0::2], zr.real, atol=1e-12)
    assert np.allclose(y[..., 1::2], zr.imag, atol=1e-12)


def test_rope_preserves_pair_norms_and_relative_logits():
    rng = np.random.default_rng(8)
    d = 64
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    qn = np.hypot(q[..., 0::2], q[..., 1::2])
    for p in (0, 5, 1000, 123457):
        y = O.rope(q, np.array([p]), 1e4)
        assert np.allclose(np.hypot(y[..., 0::2], y[..., 1::2]), qn, atol=1e-12)
    # q_i . k_j depends only on i - j
    dots = []
    for i, j in [(10, 3), (17, 10), (100007, 100000)]:
        dots.append(float((O.rope(q, np.array([i]), 1e4) * O.rope(k, np.array([j]), 1e4)).sum()))
    assert np.allclose(dots, dots[0], atol=1e-9)


@pytest.mark.parametrize("theta,d_h,s", [(1e4, 64, 1.0), (1e6, 128, 1.0), (1e6, 128, 4.0)])
def test_no_wavelength_near_an_integer(theta, d_h, s):
    # the floor() in the cutoff is robust: every w_c sits >= 1e-6 from an integer
    w = O.wavelengths(theta, d_h, s)
    assert np.min(np.abs(w - np.round(w))) > 1e-6
