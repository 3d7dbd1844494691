"""GPU parity of wp_prefill (and the RoPE -> prefill path) against the oracle.

O: max-abs <= 2e-2 and mean-abs <= 2e-3 element by element.  Tile-class
counters: bit-exact against the oracle's classifier on the kernel's grid."""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
from gpu_util import (Timer, bf16_to_np, bits_to_dev, compare, dev, oracle_prefill_rows,
                      prefill_inputs, say, separation, to_f64)

pytestmark = pytest.mark.gpu


def _expected_counts(n, d_h, G, cut, copies):
    BM, BN = W.prefill_tiling(d_h, G)
    c, v = O.prefill_tile_counts(n, BM, BN, np.asarray(cut))
    return (np.concatenate([c.ravel(), [v]]) * copies).astype(np.int64)


def _counters(d_h, G):
    return torch.zeros(3 * (d_h // G) + 1, dtype=torch.int64, device=dev())


# --------------------------------------------------------------------------
# small shapes, all rows: ragged tails, GQA ratios 1/2/3/4/8, d_h 64/128,
# G 16/32, thetas small enough that skip / partial / full all occur, and one
# where far keys lose every group (logit exactly 0, key kept).
# inputs are used directly as the rotated q, k.
# --------------------------------------------------------------------------
SMALL = [
    # B, n, Hq, Hkv, d, G, theta, s
    (1, 1, 1, 1, 64, 16, 1e4, 1.0),
    (2, 100, 4, 2, 64, 32, 100.0, 1.0),
    (1, 777, 3, 1, 128, 16, 1e3, 1.0),
    (1, 1000, 8, 1, 128, 32, 1e4, 1.0),
    (1, 513, 16, 2, 128, 16, 1e6, 4.0),
    (1, 300, 4, 4, 64, 16, 30.0, 1.0),
    (3, 161, 8, 2, 128, 16, 300.0, 1.0),
    (1, 500, 32, 1, 128, 16, 100.0, 1.0),       # MQA: 32 query heads on one kv head
]


@pytest.mark.parametrize("B,n,Hq,Hkv,d,G,theta,s", SMALL)
@pytest.mark.parametrize("dense", [False, True])
def test_prefill_small_all_rows(B, n, Hq, Hkv, d, G, theta, s, dense):
    say("prefill B=%d n=%d Hq=%d Hkv=%d d=%d G=%d theta=%g s=%g dense=%s"
        % (B, n, Hq, Hkv, d, G, theta, s, dense))
    seed = 1000 + n + Hq
    q = synth.normal_bits(seed, 0, B * n, (Hq, d))
    k = synth.normal_bits(seed, 1, B * n, (Hkv, d))
    v = synth.normal_bits(seed, 2, B * n, (Hkv, d))
    cut = [int(c) for c in O.group_cutoffs(theta, d, G, s)]
    qt, kt, vt = (bits_to_dev(x, (B, n, x.shape[1], d)) for x in (q, k, v))
    cnt = _counters(d, G)
    o = torch.full((B, n, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev())
    o, lse = W.prefill(qt, kt, vt, None if dense else cut, G, dense=dense, return_lse=True,
                       counters=cnt, out=o)
    torch.cuda.synchronize()
    got = bf16_to_np(o).reshape(B, n, Hq, d)
    got_lse = lse.cpu().numpy()
    dim_cut = O.dim_cutoffs_dense(d) if dense else O.dim_cutoffs_grouped(np.array(cut), G)
    for b in range(B):
        sl = slice(b * n, (b + 1) * n)
        ref, ref_lse = O.prefill(to_f64(q[sl]), to_f64(k[sl]), to_f64(v[sl]), dim_cut, return_lse=True)
        compare(got[b], ref, "O b=%d" % b)
        compare(got_lse[b].T, ref_lse, "LSE b=%d" % b)
    exp = _expected_counts(n, d, G, [O.NEVER] * (d // G) if dense else cut, B * Hq)
    assert np.array_equal(cnt.cpu().numpy(), exp), (cnt.cpu().numpy(), exp)


# the v_mfma_f32_16x16x32_bf16 kernel (d_h 128, G 32): the same checks on
# every row, ragged tails, GQA ratios 1/2/3/4/8/32, small thetas (skip,
# partial, full and fully pruned keys), dense
SMALL_MFMA16 = [
    # B, n, Hq, Hkv, theta, s
    (1, 1, 1, 1, 1e4, 1.0),
    (2, 100, 4, 2, 30.0, 1.0),
    (1, 777, 3, 1, 1e3, 1.0),
    (1, 1000, 8, 1, 300.0, 1.0),
    (1, 513, 16, 2, 1e6, 4.0),
    (3, 161, 8, 2, 100.0, 1.0),
    (1, 500, 32, 1, 1e4, 1.0),
]


@pytest.mark.parametrize("B,n,Hq,Hkv,theta,s", SMALL_MFMA16)
@pytest.mark.parametrize("dense", [False, True])
def test_prefill_mfma16_all_rows(B, n, Hq, Hkv, theta, s, dense):
    d, G = 128, 32
    say("prefill 16x16x32 B=%d n=%d Hq=%d Hkv=%d theta=%g s=%g dense=%s" % (B, n, Hq, Hkv, theta, s, dense))
    seed = 1500 + n + Hq
    q = synth.normal_bits(seed, 0, B * n, (Hq, d))
    k = synth.normal_bits(seed, 1, B * n, (Hkv, d))
    v = synth.normal_bits(seed, 2, B * n, (Hkv, d))
    cut = [int(c) for c in O.group_cutoffs(theta, d, G, s)]
    qt, kt, vt = (bits_to_dev(x, (B, n, x.shape[1], d)) for x in (q, k, v))
    cnt = _counters(d, G)
    o = torch.full((B, n, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev())
    o, lse = W.prefill(qt, kt, vt, None if dense else cut, G, dense=dense, return_lse=True,
                       counters=cnt, out=o, variant="mfma16x16x32")
    o32 = W.prefill(qt, kt, vt, None if dense else cut, G, dense=dense)
    torch.cuda.synchronize()
    got = bf16_to_np(o).reshape(B, n, Hq, d)
    got_lse = lse.cpu().numpy()
    dim_cut = O.dim_cutoffs_dense(d) if dense else O.dim_cutoffs_grouped(np.array(cut), G)
    for b in range(B):
        sl = slice(b * n, (b + 1) * n)
        ref, ref_lse = O.prefill(to_f64(q[sl]), to_f64(k[sl]), to_f64(v[sl]), dim_cut, return_lse=True)
        compare(got[b], ref, "O b=%d" % b)
        compare(got_lse[b].T, ref_lse, "LSE b=%d" % b)
    exp = _expected_counts(n, d, G, [O.NEVER] * (d // G) if dense else cut, B * Hq)
    assert np.array_equal(cnt.cpu().numpy(), exp), (cnt.cpu().numpy(), exp)
    # the two MFMA shapes differ only in summation order
    diff = (o.float() - o32.float()).abs().max().item()
    say("  vs the 32x32x16 kernel: max-abs %.3e" % diff)
    assert diff <= 2e-2


def test_prefill_deterministic_and_strided():
    B, n, Hq, Hkv, d, G = 1, 700, 8, 2, 128, 16
    q = synth.normal_bits(5, 0, B * n, (Hq, d))
    k = synth.normal_bits(5, 1, B * n, (Hkv, d))
    v = synth.normal_bits(5, 2, B * n, (Hkv, d))
    cut = [int(c) for c in O.group_cutoffs(1e4, d, G)]
    qt, kt, vt = (bits_to_dev(x, (B, n, x.shape[1], d)) for x in (q, k, v))
    o1 = W.prefill(qt, kt, vt, cut, G)
    o2 = W.prefill(qt, kt, vt, cut, G)
    # k and v as views into one packed [B, n, 2*Hkv, d] tensor; o into a wider buffer
    kv = torch.cat([kt, vt], dim=2)
    big = torch.zeros((B, n, Hq + 4, d), dtype=torch.bfloat16, device=dev())
    o3 = W.prefill(qt, kv[:, :, :Hkv], kv[:, :, Hkv:], cut, G, out=big[:, :, 2:2 + Hq])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(o1, o3)
    assert torch.count_nonzero(big[:, :, :2]) == 0 and torch.count_nonzero(big[:, :, 2 + Hq:]) == 0


# --------------------------------------------------------------------------
# the workloads: raw inputs -> wp_rope_apply -> wp_prefill, oracle from the raw
# inputs (float64 RoPE, grouped rule)
# --------------------------------------------------------------------------
def _run_workload(name, nrows_override=None, sep_rows=0, e2e_rows=None, variant=None):
    """Counters over the whole grid; O on the oracle's rows (nrows_override
    or the workload's own count, 0 = every row) against the bf16-in oracle;
    the end-to-end comparison against float64 RoPE on those rows, or on
    e2e_rows of them picked evenly."""
    w = synth.WORKLOADS[name]
    say("workload %s: B=%d n=%d Hq=%d Hkv=%d d=%d G=%d theta=%g s=%g"
        % (name, w.B, w.n, w.Hq, w.Hkv, w.d_h, w.G, w.theta, w.pos_scale))
    with Timer("inputs"):
        q_raw, k_raw, v_bits, _ = prefill_inputs(w)
    shape_q = (w.B, w.n, w.Hq, w.d_h)
    shape_k = (w.B, w.n, w.Hkv, w.d_h)
    cut = W.group_cutoffs(w.theta, w.d_h, w.G, w.pos_scale)
    assert cut == [int(c) for c in O.group_cutoffs(w.theta, w.d_h, w.G, w.pos_scale)]
    with Timer("gpu rope+prefill"):
        if w.fp32_inputs:
            qd = torch.from_numpy(q_raw).reshape(shape_q).to(dev())
            kd = torch.from_numpy(k_raw).reshape(shape_k).to(dev())
        else:
            qd = bits_to_dev(q_raw, shape_q)
            kd = bits_to_dev(k_raw, shape_k)
        vd = bits_to_dev(v_bits, shape_k)
        qr = W.rope_apply(qd, w.theta, w.pos_scale)
        kr = W.rope_apply(kd, w.theta, w.pos_scale)
        del qd, kd
        cnt = _counters(w.d_h, w.G)
        o = W.prefill(qr, kr, vd, cut, w.G, counters=cnt, variant=variant)
        torch.cuda.synchronize()
    exp = _expected_counts(w.n, w.d_h, w.G, cut, w.B * w.Hq)
    got_cnt = cnt.cpu().numpy()
    say("  counters", got_cnt.tolist())
    assert np.array_equal(got_cnt, exp), (got_cnt, exp)

    nrows = nrows_override if nrows_override is not None else w.oracle_rows
    special = [c + e for c in cut for e in (0, 1)]
    rows = np.arange(w.n) if nrows == 0 else synth.sample_rows(w.n, nrows, w.seed, special)
    got = bf16_to_np(o[0, torch.from_numpy(rows).to(dev())]).reshape(len(rows), w.Hq, w.d_h)
    del o, qr, kr, vd
    q_rows = q_raw[rows]
    # G = 2 is checked against the oracle's exact per-channel rule itself
    dim_cut = (O.dim_cutoffs_exact(w.theta, w.d_h, w.pos_scale) if w.G == 2
               else O.dim_cutoffs_grouped(np.array(cut), w.G))
    with Timer("oracle %d rows, bf16-in" % len(rows)):
        # bf16-in reference: the oracle's rotated q, k rounded to bf16, the
        # precision the attention kernel consumes
        ref_b = oracle_prefill_rows(w, q_rows, k_raw, v_bits, rows, dim_cut, bf16_in=True)
    compare(got, ref_b, "%s O vs bf16-in oracle (%d rows)" % (name, len(rows)))
    if e2e_rows is not None and e2e_rows < len(rows):
        pick = np.linspace(0, len(rows) - 1, e2e_rows).astype(int)
        rows, q_rows, got, ref_b = rows[pick], q_rows[pick], got[pick], ref_b[pick]
    with Timer("oracle %d rows, float64 RoPE" % len(rows)):
        ref = oracle_prefill_rows(w, q_rows, k_raw, v_bits, rows, dim_cut)
    # end to end against float64 RoPE: the gate plus the shift that rounding
    # the rotated inputs to bf16 alone causes in the oracle
    shift = np.abs(ref_b - ref)
    say("  oracle shift from bf16 rotated inputs: max %.3e mean %.3e" % (shift.max(), shift.mean()))
    compare(got, ref, "%s O vs fp64-RoPE oracle" % name,
            max_abs=2e-2 + float(shift.max()), mean_abs=2e-3 + float(shift.mean()))
    if sep_rows:
        sub = rows[np.linspace(0, len(rows) - 1, sep_rows).astype(int)]
        pick = np.searchsorted(rows, sub)
        dense = oracle_prefill_rows(w, q_rows[pick], k_raw, v_bits, sub, O.dim_cutoffs_dense(w.d_h))
        exact = oracle_prefill_rows(w, q_rows[pick], k_raw, v_bits, sub,
                                    O.dim_cutoffs_exact(w.theta, w.d_h, w.pos_scale))
        separation(ref[pick], dense, "grouped vs dense")
        separation(ref[pick], exact, "grouped vs exact")
    return got, ref, rows


def test_workload_tiny256():
    got, ref, rows = _run_workload("tiny256", sep_rows=256)
    # the same GPU output against the oracle on the bf16-rounded q, k
    w = synth.WORKLOADS["tiny256"]
    q_raw, k_raw, v_bits, _ = prefill_inputs(w)
    qb = synth.bf16_round(q_raw)
    kb = synth.bf16_round(k_raw)
    cut = O.group_cutoffs(w.theta, w.d_h, w.G)
    ref_b = oracle_prefill_rows(w, qb[rows], kb, v_bits, rows, O.dim_cutoffs_grouped(cut, w.G))
    compare(got, ref_b, "tiny256 O vs oracle on bf16 q,k")


@pytest.mark.timeout(600)
def test_workload_prefill4k():
    # every one of the 4096 rows against the bf16-in oracle; the end-to-end
    # float64-RoPE comparison on 384 of them
    _run_workload("prefill4k", nrows_override=0, sep_rows=32, e2e_rows=384)


@pytest.mark.parametrize("name", ["prefill32k_g16", "prefill32k_g32"])
def test_workload_prefill32k(name):
    _run_workload(name, sep_rows=16)


def test_workload_prefill32k_g32_mfma16():
    _run_workload("prefill32k_g32", variant="mfma16x16x32")


def test_workload_prefill32k_exact():
    _run_workload("prefill32k_exact", sep_rows=16)


def test_workload_prefill128k_scaled():
    _run_workload("prefill128k_s4")


def test_prefill_kv_past_2gib():
    """K and V sequences past what one 32-bit buffer resource spans: 6144
    tokens at a 512 KB token stride (views of one head out of 2048), so the
    last key sits 3 GiB past the first (each 64-key tile is read through its
    own resources).  Sampled rows against the oracle, counters bit-exact."""
    n, Hq, Hkv, Hall, d, G, theta = 6144, 4, 1, 2048, 128, 16, 1e4
    say("prefill past 2 GiB: n=%d token stride %d bytes" % (n, Hall * d * 2))
    assert (n - 1) * Hall * d * 2 > 3 * 2 ** 30 - 2 ** 20
    q = synth.normal_bits(91, 0, n, (Hq, d))
    k = synth.normal_bits(91, 1, n, (Hkv, d))
    v = synth.normal_bits(91, 2, n, (Hkv, d))
    qt = bits_to_dev(q, (1, n, Hq, d))
    kbig = torch.zeros((1, n, Hall, d), dtype=torch.bfloat16, device=dev())
    vbig = torch.zeros((1, n, Hall, d), dtype=torch.bfloat16, device=dev())
    kbig[:, :, Hall - 1:] = bits_to_dev(k, (1, n, Hkv, d))       # the last head: the far end of the buffer
    vbig[:, :, Hall - 1:] = bits_to_dev(v, (1, n, Hkv, d))
    cut = W.group_cutoffs(theta, d, G)
    cnt = _counters(d, G)
    o = W.prefill(qt, kbig[:, :, Hall - 1:], vbig[:, :, Hall - 1:], cut, G, counters=cnt)
    torch.cuda.synchronize()
    del kbig, vbig
    rows = synth.sample_rows(n, 96, 91, [c + e for c in cut for e in (0, 1)])
    got = bf16_to_np(o[0, torch.from_numpy(rows).to(dev())]).reshape(len(rows), Hq, d)
    ref = O.prefill(to_f64(q), to_f64(k), to_f64(v), O.dim_cutoffs_grouped(np.array(cut), G), rows=rows)
    compare(got, ref, "prefill largest span (%d rows)" % len(rows))
    assert np.array_equal(cnt.cpu().numpy(), _expected_counts(n, d, G, cut, Hq))
