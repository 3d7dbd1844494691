"""GPU parity of prefill, decode and the backward with cutoff tables from
general sources: a per-channel scaled frequency vector, alpha != 2, and
truncation of only the first channels (wp_cutoffs_from_freqs).  The kernels take any
non-decreasing table; these cases check the table end to end against the
oracle's own general-cutoff path (all rows, max-abs 2e-2 / mean-abs 2e-3,
tile counters bit-exact)."""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
import bwd_bound as BB
from gpu_util import bf16_to_np, bits_to_dev, compare, dev, say, to_f64

pytestmark = pytest.mark.gpu


def _ramp_scaled(theta, d_h, s, lo=0.25, hi=0.75):
    """First `lo` of the channels unscaled, last 1-hi divided by s, linear in
    between: a per-channel scaled schedule (the frequencies the model would
    rotate with)."""
    n = d_h // 2
    f = O.frequencies(theta, d_h)
    t = np.clip((np.arange(n) / (n - 1) - lo) / (hi - lo), 0.0, 1.0)
    return f / (1.0 + t * (s - 1.0))


# name, d_h, G, frequency vector, alpha, truncated channels
CASES = [
    ("ramp s=8 alpha=1.5", 128, 16, lambda: _ramp_scaled(1e3, 128, 8.0), 1.5, None),
    ("theta=300 alpha=3 first 20 ch", 64, 16, lambda: O.frequencies(300.0, 64), 3.0, 20),
    ("theta=1e3 alpha=0.5", 128, 32, lambda: O.frequencies(1e3, 128), 0.5, None),
]


def _table(d, G, freqs, alpha, trunc):
    n_ch = d // 2
    k = n_ch if trunc is None else trunc
    got = W.cutoffs_from_freqs(list(freqs), G, alpha, k)
    ref = [int(v) for v in O.group_max(O.cutoffs_from_freqs(freqs, alpha, k), G)]
    assert got == ref, (got, ref)
    return got


@pytest.mark.parametrize("name,d,G,fv,alpha,trunc", CASES)
def test_prefill_general_table(name, d, G, fv, alpha, trunc):
    B, n, Hq, Hkv = 1, 600, 8, 2
    say("prefill general table: %s n=%d" % (name, n))
    cut = _table(d, G, fv(), alpha, trunc)
    q = synth.normal_bits(31, 0, B * n, (Hq, d))
    k = synth.normal_bits(31, 1, B * n, (Hkv, d))
    v = synth.normal_bits(31, 2, B * n, (Hkv, d))
    qt, kt, vt = (bits_to_dev(x, (B, n, x.shape[1], d)) for x in (q, k, v))
    cnt = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    o = W.prefill(qt, kt, vt, cut, G, counters=cnt)
    torch.cuda.synchronize()
    got = bf16_to_np(o).reshape(n, Hq, d)
    ref = O.prefill(to_f64(q), to_f64(k), to_f64(v), O.dim_cutoffs_grouped(np.array(cut), G))
    compare(got, ref, "O %s" % name)
    BM, BN = W.prefill_tiling(d, G)
    c, vis = O.prefill_tile_counts(n, BM, BN, np.asarray(cut))
    exp = (np.concatenate([c.ravel(), [vis]]) * B * Hq).astype(np.int64)
    assert np.array_equal(cnt.cpu().numpy(), exp)


@pytest.mark.parametrize("name,d,G,fv,alpha,trunc", CASES)
def test_decode_general_table(name, d, G, fv, alpha, trunc):
    B, Lmax, Hq, Hkv = 2, 1500, 8, 2
    lens = [1500, 777]
    say("decode general table: %s lens=%s" % (name, lens))
    cut = _table(d, G, fv(), alpha, trunc)
    q = synth.normal_bits(32, 0, B, (Hq, d))
    kc = synth.normal_bits(32, 1, B * Lmax, (Hkv, d))
    vc = synth.normal_bits(32, 2, B * Lmax, (Hkv, d))
    qt = bits_to_dev(q, (B, Hq, d))
    kt = bits_to_dev(kc, (B, Lmax, Hkv, d))
    vt = bits_to_dev(vc, (B, Lmax, Hkv, d))
    cl = torch.tensor(lens, dtype=torch.int32, device=dev())
    qp = torch.tensor(lens, dtype=torch.int32, device=dev())
    o = W.decode(qt, kt, vt, cl, qp, cut, G)
    torch.cuda.synchronize()
    got = bf16_to_np(o)
    dim_cut = O.dim_cutoffs_grouped(np.array(cut), G)
    for b in range(B):
        sl = slice(b * Lmax, (b + 1) * Lmax)
        ref = O.decode(to_f64(q[b]), to_f64(kc[sl]), to_f64(vc[sl]), lens[b], lens[b], dim_cut)
        compare(got[b], ref, "decode %s b=%d" % (name, b))


@pytest.mark.parametrize("name,d,G,fv,alpha,trunc", CASES)
def test_backward_general_table(name, d, G, fv, alpha, trunc):
    """The backward pass with the same general tables: dQ, dK, dV against the
    oracle's backward on every element (the rounding bound of
    tests/bwd_bound.py element by element, mean-abs 2e-3, mean-abs <= 4e-3
    of the mean magnitude)."""
    B, n, Hq, Hkv = 1, 300, 4, 2
    say("backward general table: %s n=%d" % (name, n))
    cut = _table(d, G, fv(), alpha, trunc)
    x = [synth.normal_bits(37, t, B * n, (h, d)) for t, h in ((0, Hq), (1, Hkv), (2, Hkv), (3, Hq))]
    qt, kt, vt, gt = (bits_to_dev(a, (B, n, a.shape[1], d)) for a in x)
    o, lse = W.prefill(qt, kt, vt, cut, G, return_lse=True)
    grads = W.prefill_backward(qt, kt, vt, o, gt, lse, cut, G)
    torch.cuda.synchronize()
    x64 = [to_f64(a) for a in x]
    dim_cut = O.dim_cutoffs_grouped(np.array(cut), G)
    ref = O.prefill_backward(*x64, dim_cut)
    R = BB.backward_terms(*x64, dim_cut)
    for nm, gg, rr, RR in zip(("dQ", "dK", "dV"), grads, ref, R):
        got = bf16_to_np(gg).reshape(rr.shape)
        err = np.abs(got - rr)
        BB.check(got, rr, RR, nm, say)
        assert err.mean() <= 2e-3 and err.mean() <= 4e-3 * np.abs(rr).mean(), (nm, err.mean())
