"""GPU parity of the fine-group kernels: G = 2 (every channel its own cutoff,
the exact per-channel rule), G = 4 and G = 8, in prefill and decode.

With G = 2 the expected values come from the oracle's exact rule
(dim_cutoffs_exact: one cutoff per RoPE channel), not from a grouped table,
so the test also checks that G = 2 grouping is the exact rule.  Small
thetas put many channels in the partial class on the same tile, so the
masked per-group MFMAs inside one 16-dim step are exercised; sizes span
several tiles with ragged tails.  Tile counters are compared bit-exactly
with the oracle's classifier (max-abs 2e-2 / mean-abs 2e-3 on outputs)."""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
from gpu_util import bf16_to_np, bits_to_dev, compare, dev, say, to_f64

pytestmark = pytest.mark.gpu


def _dim_cut(theta, d, G):
    if G == 2:
        return O.dim_cutoffs_exact(theta, d)
    return O.dim_cutoffs_grouped(O.group_cutoffs(theta, d, G), G)


# d_h, G, theta, n, Hq, Hkv
PREFILL = [
    (128, 2, 1e4, 600, 8, 2),
    (128, 2, 300.0, 333, 4, 4),
    (64, 2, 1e3, 517, 8, 1),
    (128, 4, 1e3, 257, 4, 1),
    (128, 8, 1e6, 1000, 8, 2),
    (64, 4, 100.0, 200, 2, 2),
    (64, 8, 3e4, 700, 4, 2),
]


@pytest.mark.parametrize("d,G,theta,n,Hq,Hkv", PREFILL)
def test_prefill_fine_groups(d, G, theta, n, Hq, Hkv):
    B = 1
    say("prefill fine groups: d=%d G=%d theta=%g n=%d Hq=%d Hkv=%d" % (d, G, theta, n, Hq, Hkv))
    cut = W.group_cutoffs(theta, d, G)
    seed = 70 + G + n
    q = synth.normal_bits(seed, 0, B * n, (Hq, d))
    k = synth.normal_bits(seed, 1, B * n, (Hkv, d))
    v = synth.normal_bits(seed, 2, B * n, (Hkv, d))
    qt, kt, vt = (bits_to_dev(x, (B, n, x.shape[1], d)) for x in (q, k, v))
    cnt = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    o = W.prefill(qt, kt, vt, cut, G, counters=cnt)
    torch.cuda.synchronize()
    got = bf16_to_np(o).reshape(n, Hq, d)
    ref = O.prefill(to_f64(q), to_f64(k), to_f64(v), _dim_cut(theta, d, G))
    compare(got, ref, "O d=%d G=%d theta=%g" % (d, G, theta))
    BM, BN = W.prefill_tiling(d, G)
    c, vis = O.prefill_tile_counts(n, BM, BN, np.asarray(cut))
    exp = (np.concatenate([c.ravel(), [vis]]) * B * Hq).astype(np.int64)
    assert np.array_equal(cnt.cpu().numpy(), exp)
    # the plain-call path (no counters) gives the same bits
    o2 = W.prefill(qt, kt, vt, cut, G)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))


# d_h, G, theta, Lmax, lens, Hq, Hkv
DECODE = [
    (128, 2, 1e4, 1500, [1500, 777], 8, 2),
    (64, 2, 300.0, 900, [900, 1], 4, 1),
    (128, 4, 1e3, 2100, [2100, 64], 16, 4),
    (128, 8, 1e5, 3000, [3000, 2999], 8, 8),
]


@pytest.mark.parametrize("d,G,theta,Lmax,lens,Hq,Hkv", DECODE)
def test_decode_fine_groups(d, G, theta, Lmax, lens, Hq, Hkv):
    B = len(lens)
    say("decode fine groups: d=%d G=%d theta=%g lens=%s Hq=%d Hkv=%d" % (d, G, theta, lens, Hq, Hkv))
    cut = W.group_cutoffs(theta, d, G)
    seed = 90 + G + Lmax
    q = synth.normal_bits(seed, 0, B, (Hq, d))
    kc = synth.normal_bits(seed, 1, B * Lmax, (Hkv, d))
    vc = synth.normal_bits(seed, 2, B * Lmax, (Hkv, d))
    qt = bits_to_dev(q, (B, Hq, d))
    kt = bits_to_dev(kc, (B, Lmax, Hkv, d))
    vt = bits_to_dev(vc, (B, Lmax, Hkv, d))
    cl = torch.tensor(lens, dtype=torch.int32, device=dev())
    qp = torch.tensor(lens, dtype=torch.int32, device=dev())
    cnt = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    o = W.decode(qt, kt, vt, cl, qp, cut, G, counters=cnt)
    torch.cuda.synchronize()
    got = bf16_to_np(o)
    dim_cut = _dim_cut(theta, d, G)
    exp = np.zeros(3 * (d // G) + 1, dtype=np.int64)
    for b in range(B):
        sl = slice(b * Lmax, (b + 1) * Lmax)
        ref = O.decode(to_f64(q[b]), to_f64(kc[sl]), to_f64(vc[sl]), lens[b], lens[b], dim_cut)
        compare(got[b], ref, "decode d=%d G=%d b=%d" % (d, G, b))
        c, vis = O.decode_tile_counts(lens[b], lens[b], W.decode_tiling(d, G), np.asarray(cut))
        exp += (np.concatenate([c.ravel(), [vis]]) * Hkv).astype(np.int64)   # once per kv head
    got_cnt = cnt.cpu().numpy()
    assert np.array_equal(got_cnt, exp), (got_cnt, exp)
