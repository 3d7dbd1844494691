"""GPU parity of wp_prefill_backward against the oracle's backward pass.

The GPU gradients use the GPU forward's bf16 O and float LSE, bf16 P and dS
MFMA operands and float accumulation, and are rounded to bf16; the oracle
works in float64 from the same bf16 inputs.  Gate, element by element: the
bound that tests/bwd_bound.py derives from those roundings,
|gpu - oracle| <= u |oracle| + 8 u sqrt(R) + 1e-6 with u = 2^-8 and R the
sum of the squared rounded terms of that element (checked against a float64
emulation of the roundings, and shown to catch planted mistakes, in
tests/test_bwd_bound.py).  Per tensor also: mean-abs error <= 4e-3 of the
mean magnitude (emulating the roundings gives 2.1e-3: bf16 output rounding
alone 1.4e-3) and mean-abs <= 2e-3 (the forward output's gate).
"""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
import bwd_bound as BB
from gpu_util import Timer, bf16_to_np, bits_to_dev, dev, say, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    # B, n, Hq, Hkv, d, G, theta, dense
    (1, 1, 1, 1, 64, 16, 1e4, False),
    (1, 100, 2, 1, 64, 16, 30.0, False),
    (2, 300, 4, 2, 128, 16, 300.0, False),
    (1, 257, 8, 2, 128, 32, 1e3, False),
    (1, 513, 4, 4, 64, 32, 100.0, False),
    (1, 200, 4, 1, 128, 16, 1e4, True),
    (1, 161, 6, 2, 128, 16, 50.0, False),
    (1, 2048, 4, 1, 128, 16, 1e4, False),          # many tiles at a realistic theta
    # fine groups: G = 2 is the exact per-channel rule; small thetas put many
    # channels in the partial class on one tile
    (1, 300, 4, 2, 128, 2, 300.0, False),
    (2, 257, 8, 2, 128, 4, 1e3, False),
    (1, 400, 4, 1, 128, 8, 50.0, False),
    (1, 333, 4, 4, 64, 2, 100.0, False),
    (1, 200, 2, 1, 64, 8, 1e4, False),
    (1, 1000, 8, 2, 128, 2, 1e4, False),
]


def _rel_errors(got, ref):
    # a single-token sequence has dQ = dK = 0 exactly: floor the scale
    scale = max(np.abs(ref).mean(), 1e-3)
    err = np.abs(got - ref)
    return err.max() / scale, err.mean() / scale


@pytest.mark.parametrize("B,n,Hq,Hkv,d,G,theta,dense", CASES)
def test_backward_matches_oracle(B, n, Hq, Hkv, d, G, theta, dense):
    say("backward B=%d n=%d Hq=%d Hkv=%d d=%d G=%d theta=%g dense=%s" % (B, n, Hq, Hkv, d, G, theta, dense))
    seed = 4000 + n + Hq
    q = synth.normal_bits(seed, 0, B * n, (Hq, d))
    k = synth.normal_bits(seed, 1, B * n, (Hkv, d))
    v = synth.normal_bits(seed, 2, B * n, (Hkv, d))
    g = synth.normal_bits(seed, 3, B * n, (Hq, d))
    cut = [int(c) for c in O.group_cutoffs(theta, d, G)]
    qt, kt, vt, gt = (bits_to_dev(x, (B, n, x.shape[1], d)) for x in (q, k, v, g))
    o, lse = W.prefill(qt, kt, vt, None if dense else cut, G, dense=dense, return_lse=True)
    dq, dk, dv = W.prefill_backward(qt, kt, vt, o, gt, lse, None if dense else cut, G, dense=dense)
    torch.cuda.synchronize()
    got = [bf16_to_np(x).reshape(B, n, x.shape[2], d) for x in (dq, dk, dv)]
    if dense:
        dim_cut = O.dim_cutoffs_dense(d)
    elif G == 2:
        dim_cut = O.dim_cutoffs_exact(theta, d)      # G = 2 against the exact rule itself
    else:
        dim_cut = O.dim_cutoffs_grouped(np.array(cut), G)
    for b in range(B):
        sl = slice(b * n, (b + 1) * n)
        x64 = [to_f64(x[sl]) for x in (q, k, v, g)]
        ref = O.prefill_backward(*x64, dim_cut)
        R = BB.backward_terms(*x64, dim_cut)
        for name, gg, rr, RR in zip(("dQ", "dK", "dV"), got, ref, R):
            mx, mean = _rel_errors(gg[b], rr)
            say("  b=%d %s: relative to mean |ref| = %.3g: max %.2e, mean %.2e"
                % (b, name, np.abs(rr).mean(), mx, mean))
            BB.check(gg[b], rr, RR, "b=%d %s" % (b, name), say)
            assert np.abs(gg[b] - rr).mean() <= 2e-3, name
            assert mean <= 4e-3, (name, mean)


def test_backward_deterministic():
    B, n, Hq, Hkv, d, G = 1, 400, 4, 1, 128, 16
    x = [synth.normal_bits(77, t, B * n, (h, d)) for t, h in ((0, Hq), (1, Hkv), (2, Hkv), (3, Hq))]
    qt, kt, vt, gt = (bits_to_dev(a, (B, n, a.shape[1], d)) for a in x)
    cut = W.group_cutoffs(300.0, d, G)
    o, lse = W.prefill(qt, kt, vt, cut, G, return_lse=True)
    r1 = W.prefill_backward(qt, kt, vt, o, gt, lse, cut, G)
    r2 = W.prefill_backward(qt, kt, vt, o, gt, lse, cut, G)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_workload_32k():
    """The 32K prefill shape (32/8 heads, d_h 128, theta 1e6, G 16) through
    the three backward kernels in the launch configuration the bench times,
    checked on a sample: dQ at 24 sampled rows and the last 40 rows, dK and
    dV at the last 40 keys (complete from those rows, by causality)."""
    n, Hq, Hkv, d, G, theta = 32768, 32, 8, 128, 16, 1e6
    seed, tail = 6100, 40
    say("backward workload: n=%d Hq=%d Hkv=%d d=%d G=%d theta=%g" % (n, Hq, Hkv, d, G, theta))
    with Timer("inputs"):
        q = synth.normal_bits(seed, 0, n, (Hq, d))
        k = synth.normal_bits(seed, 1, n, (Hkv, d))
        v = synth.normal_bits(seed, 2, n, (Hkv, d))
        g = synth.normal_bits(seed, 3, n, (Hq, d))
    cut = [int(c) for c in O.group_cutoffs(theta, d, G)]
    with Timer("gpu forward + backward"):
        qt, kt, vt, gt = (bits_to_dev(x, (1, n, x.shape[1], d)) for x in (q, k, v, g))
        o, lse = W.prefill(qt, kt, vt, cut, G, return_lse=True)
        dq, dk, dv = W.prefill_backward(qt, kt, vt, o, gt, lse, cut, G)
        torch.cuda.synchronize()
    key_from = n - tail
    special = [c + e for c in cut for e in (0, 1)]
    rows = np.union1d(synth.sample_rows(n, 24, seed, special), np.arange(key_from, n))
    ridx = torch.from_numpy(rows).to(dev())
    got_dq = bf16_to_np(dq[0, ridx]).reshape(len(rows), Hq, d)
    got_dk = bf16_to_np(dk[0, key_from:]).reshape(tail, Hkv, d)
    got_dv = bf16_to_np(dv[0, key_from:]).reshape(tail, Hkv, d)
    del o, lse, dq, dk, dv, qt, kt, vt, gt
    dim_cut = O.dim_cutoffs_grouped(np.array(cut), G)
    x64 = [to_f64(x) for x in (q, k, v, g)]
    with Timer("oracle %d rows" % len(rows)):
        ref = O.prefill_backward_rows(*x64, dim_cut, rows, key_from)
    with Timer("error bound terms"):
        R = BB.backward_terms(*x64, dim_cut, rows, key_from)
    # the tail keys get gradient from at most 40 rows, so their magnitudes
    # are small (~4e-4): the relative gate uses the tensor's own mean, no floor
    for name, gg, rr, RR in zip(("dQ rows", "dK tail", "dV tail"), (got_dq, got_dk, got_dv), ref, R):
        err = np.abs(gg - rr)
        scale = np.abs(rr).mean()
        say("  %s: relative to mean |ref| = %.3g: %.2e / %.2e" % (name, scale, err.max() / scale, err.mean() / scale))
        BB.check(gg, rr, RR, name, say)
        assert err.mean() <= 2e-3, (name, err.mean())
        assert err.mean() <= 4e-3 * scale, (name, err.mean() / scale)


def test_backward_strided_views():
    """q, k, v as views into one packed [B, n, Hq + 2 Hkv, d] projection
    output, dO as a view into a wider tensor, and dQ, dK, dV written into one
    packed gradient buffer: bit-identical to the contiguous call, the
    buffer's padding untouched."""
    B, n, Hq, Hkv, d, G = 2, 333, 8, 2, 128, 16
    x = [synth.normal_bits(53, t, B * n, (h, d)) for t, h in ((0, Hq), (1, Hkv), (2, Hkv), (3, Hq))]
    qt, kt, vt, gt = (bits_to_dev(a, (B, n, a.shape[1], d)) for a in x)
    cut = W.group_cutoffs(300.0, d, G)
    o, lse = W.prefill(qt, kt, vt, cut, G, return_lse=True)
    r1 = W.prefill_backward(qt, kt, vt, o, gt, lse, cut, G)
    H = Hq + 2 * Hkv
    qkv = torch.cat([qt, kt, vt], dim=2)                  # [B, n, H, d]
    gw = torch.zeros((B, n, Hq + 2, d), dtype=torch.bfloat16, device=dev())
    gw[:, :, 1:1 + Hq] = gt
    grad = torch.zeros((B, n, H + 2, d), dtype=torch.bfloat16, device=dev())
    dq, dk, dv = (grad[:, :, 1:1 + Hq], grad[:, :, 1 + Hq:1 + Hq + Hkv], grad[:, :, 1 + Hq + Hkv:1 + H])
    r2 = W.prefill_backward(qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:], o,
                            gw[:, :, 1:1 + Hq], lse, cut, G, out=(dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.count_nonzero(grad[:, :, 0]) == 0 and torch.count_nonzero(grad[:, :, 1 + H]) == 0


def test_backward_past_2gib():
    """q, k, v and dO as head views at a 512 KB token stride, 6144 tokens:
    every input sequence reaches 3 GiB past its first row, past what one
    32-bit buffer resource spans (tiles are read through their own).  dQ at
    sampled rows and the last 48 rows, dK and dV at the last 48 keys, against
    the oracle."""
    n, Hq, Hkv, Hall, d, G, theta = 6144, 4, 1, 2048, 128, 16, 1e4
    tail = 48
    say("backward past 2 GiB: n=%d token stride %d bytes" % (n, Hall * d * 2))
    x = [synth.normal_bits(97, t, n, (h, d)) for t, h in ((0, Hq), (1, Hkv), (2, Hkv), (3, Hq))]
    views = []
    bigs = []
    for a, h in zip(x, (Hq, Hkv, Hkv, Hq)):
        big = torch.zeros((1, n, Hall, d), dtype=torch.bfloat16, device=dev())
        big[:, :, Hall - h:] = bits_to_dev(a, (1, n, h, d))
        bigs.append(big)
        views.append(big[:, :, Hall - h:])
    qt, kt, vt, gt = views
    assert (n - 1) * Hall * d * 2 > 3 * 2 ** 30 - 2 ** 20
    cut = W.group_cutoffs(theta, d, G)
    o, lse = W.prefill(qt, kt, vt, cut, G, return_lse=True)
    dq, dk, dv = W.prefill_backward(qt, kt, vt, o, gt, lse, cut, G)
    torch.cuda.synchronize()
    key_from = n - tail
    rows = np.union1d(synth.sample_rows(n, 32, 97, [c + e for c in cut for e in (0, 1)]), np.arange(key_from, n))
    got = (bf16_to_np(dq[0, torch.from_numpy(rows).to(dev())]).reshape(len(rows), Hq, d),
           bf16_to_np(dk[0, key_from:]).reshape(tail, Hkv, d), bf16_to_np(dv[0, key_from:]).reshape(tail, Hkv, d))
    del bigs, views, qt, kt, vt, gt
    x64 = [to_f64(a) for a in x]
    dim_cut = O.dim_cutoffs_grouped(np.array(cut), G)
    ref = O.prefill_backward_rows(*x64, dim_cut, rows, key_from)
    R = BB.backward_terms(*x64, dim_cut, rows, key_from)
    for nm, gg, rr, RR in zip(("dQ rows", "dK tail", "dV tail"), got, ref, R):
        err = np.abs(gg - rr)
        scale = np.abs(rr).mean()
        BB.check(gg, rr, RR, nm, say)
        assert err.mean() <= 2e-3, nm
        assert err.mean() <= 4e-3 * scale, (nm, err.mean() / scale)
