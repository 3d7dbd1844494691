"""GPU parity of wp_decode against the oracle (split-KV, suffix-K loads)."""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
from gpu_util import Timer, bf16_to_np, bits_to_dev, compare, dev, say, separation, to_f64

pytestmark = pytest.mark.gpu


def _expected(q_pos, cache_len, d_h, G, cut, Hkv):
    BN = W.decode_tiling(d_h, G)
    tot = np.zeros(3 * (d_h // G) + 1, dtype=np.int64)
    for qp, L in zip(q_pos, cache_len):
        c, v = O.decode_tile_counts(int(qp), int(L), BN, np.asarray(cut))
        tot += np.concatenate([c.ravel(), [v]]) * Hkv
    return tot


# B, Lmax, Hq, Hkv, d, G, theta, cache_len per batch, q_pos offset vs cache_len, splits
SMALL = [
    (1, 1, 1, 1, 64, 16, 1e4, [1], 0, 0),
    (3, 300, 4, 1, 64, 32, 100.0, [300, 31, 1], 0, 0),
    (2, 1000, 16, 2, 128, 16, 1e3, [1000, 333], 1, 3),
    (4, 5000, 32, 8, 128, 16, 1e4, [5000, 4097, 33, 2049], -1, 0),
    (2, 2000, 16, 1, 128, 32, 300.0, [1999, 64], 1, 1),
    (2, 700, 8, 4, 128, 16, 30.0, [700, 650], 0, 5),
]


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,d,G,theta,lens,qoff,splits", SMALL)
@pytest.mark.parametrize("dense", [False, True])
def test_decode_small(B, Lmax, Hq, Hkv, d, G, theta, lens, qoff, splits, dense):
    say("decode B=%d Lmax=%d Hq=%d Hkv=%d d=%d G=%d theta=%g lens=%s qoff=%d splits=%d dense=%s"
        % (B, Lmax, Hq, Hkv, d, G, theta, lens, qoff, splits, dense))
    seed = 2000 + Lmax + Hq
    q = synth.normal_bits(seed, 0, B, (Hq, d))
    kc = synth.normal_bits(seed, 1, B * Lmax, (Hkv, d))
    vc = synth.normal_bits(seed, 2, B * Lmax, (Hkv, d))
    # q_pos = cache_len + qoff (qoff = -1: the query's own key is the last cached one)
    q_pos = [L + qoff if L + qoff >= L - 1 else L - 1 for L in lens]
    cut = [int(c) for c in O.group_cutoffs(theta, d, G)]
    qt = bits_to_dev(q, (B, Hq, d))
    kt = bits_to_dev(kc, (B, Lmax, Hkv, d))
    vt = bits_to_dev(vc, (B, Lmax, Hkv, d))
    cl = torch.tensor(lens, dtype=torch.int32, device=dev())
    qp = torch.tensor(q_pos, dtype=torch.int32, device=dev())
    cnt = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev())
    W.decode(qt, kt, vt, cl, qp, None if dense else cut, G, dense=dense, num_splits=splits,
             counters=cnt, out=o)
    torch.cuda.synchronize()
    got = bf16_to_np(o)
    dim_cut = O.dim_cutoffs_dense(d) if dense else O.dim_cutoffs_grouped(np.array(cut), G)
    for b in range(B):
        sl = slice(b * Lmax, (b + 1) * Lmax)
        ref = O.decode(to_f64(q[b]), to_f64(kc[sl]), to_f64(vc[sl]), q_pos[b], lens[b], dim_cut)
        compare(got[b], ref, "decode b=%d L=%d" % (b, lens[b]))
    exp = _expected(q_pos, lens, d, G, [O.NEVER] * (d // G) if dense else cut, Hkv)
    assert np.array_equal(cnt.cpu().numpy(), exp), (cnt.cpu().numpy(), exp)


def test_decode_split_count_invariance():
    B, Lmax, Hq, Hkv, d, G = 2, 3000, 8, 2, 128, 16
    q = bits_to_dev(synth.normal_bits(9, 0, B, (Hq, d)), (B, Hq, d))
    k = bits_to_dev(synth.normal_bits(9, 1, B * Lmax, (Hkv, d)), (B, Lmax, Hkv, d))
    v = bits_to_dev(synth.normal_bits(9, 2, B * Lmax, (Hkv, d)), (B, Lmax, Hkv, d))
    cl = torch.tensor([3000, 2500], dtype=torch.int32, device=dev())
    qp = torch.tensor([3000, 2500], dtype=torch.int32, device=dev())
    cut = W.group_cutoffs(1e4, d, G)
    outs = [W.decode(q, k, v, cl, qp, cut, G, num_splits=s) for s in (1, 2, 7, 0)]
    again = W.decode(q, k, v, cl, qp, cut, G, num_splits=7)
    torch.cuda.synchronize()
    assert torch.equal(outs[2], again)                  # deterministic
    base = outs[0].float()
    for o in outs[1:]:
        assert (o.float() - base).abs().max().item() < 2e-2


@pytest.mark.parametrize("name", ["decode32k", "decode32k_exact"])
def test_workload_decode32k(name):
    w = synth.WORKLOADS[name]
    B, L, Hq, Hkv, d = w.B, w.n, w.Hq, w.Hkv, w.d_h
    say("workload %s: B=%d L=%d Hq=%d Hkv=%d d=%d G=%d q_pos=%d" % (name, B, L, Hq, Hkv, d, w.G, w.q_pos))
    with Timer("inputs"):
        q_raw = synth.normal_bits(w.seed, synth.TID_Q, B, (Hq, d))
        k_raw = synth.normal_bits(w.seed, synth.TID_K, B * L, (Hkv, d))
        v_bits = synth.normal_bits(w.seed, synth.TID_V, B * L, (Hkv, d))
    cut = W.group_cutoffs(w.theta, d, w.G)
    with Timer("gpu rope+decode"):
        qd = bits_to_dev(q_raw, (B, 1, Hq, d))
        kd = bits_to_dev(k_raw, (B, L, Hkv, d))
        vd = bits_to_dev(v_bits, (B, L, Hkv, d))
        qpos_t = torch.full((B,), w.q_pos, dtype=torch.int64, device=dev())
        qr = W.rope_apply(qd, w.theta, w.pos_scale, pos_start=qpos_t)[:, 0]
        kr = W.rope_apply(kd, w.theta, w.pos_scale)
        del kd
        cl = torch.full((B,), L, dtype=torch.int32, device=dev())
        qp = torch.full((B,), w.q_pos, dtype=torch.int32, device=dev())
        cnt = torch.zeros(3 * (d // w.G) + 1, dtype=torch.int64, device=dev())
        o = W.decode(qr, kr, vd, cl, qp, cut, w.G, counters=cnt)
        torch.cuda.synchronize()
    got = bf16_to_np(o)
    exp = _expected([w.q_pos] * B, [L] * B, d, w.G, cut, Hkv)
    say("  counters", cnt.cpu().numpy().tolist())
    assert np.array_equal(cnt.cpu().numpy(), exp)
    # G = 2 is checked against the oracle's exact per-channel rule itself
    dim_cut = (O.dim_cutoffs_exact(w.theta, d, w.pos_scale) if w.G == 2
               else O.dim_cutoffs_grouped(np.array(cut), w.G))
    refs, dens = [], []
    with Timer("oracle"):
        for b in range(B):
            kb = O.rope(to_f64(k_raw[b * L:(b + 1) * L]), np.arange(L), w.theta)
            qb = O.rope(to_f64(q_raw[b:b + 1]), np.array([w.q_pos]), w.theta)[0]
            vb = to_f64(v_bits[b * L:(b + 1) * L])
            refs.append(O.decode(qb, kb, vb, w.q_pos, L, dim_cut))
            if b < 2:
                dens.append(O.decode(qb, kb, vb, w.q_pos, L, O.dim_cutoffs_dense(d)))
    ref = np.stack(refs)
    compare(got, ref, "%s O" % name)
    separation(ref[:2], np.stack(dens), "grouped vs dense (2 seqs)")


def test_decode_empty_sequences():
    """A sequence with an empty cache (cache_len 0) gets o = 0 exactly and
    visits no key block; the sequences around it are unaffected."""
    B, Lmax, Hq, Hkv, d, G, theta = 4, 200, 8, 2, 128, 16, 1e3
    lens = [0, 37, 0, 200]
    say("decode empty sequences: lens=%s" % lens)
    q = synth.normal_bits(31, 0, B, (Hq, d))
    kc = synth.normal_bits(31, 1, B * Lmax, (Hkv, d))
    vc = synth.normal_bits(31, 2, B * Lmax, (Hkv, d))
    cut = W.group_cutoffs(theta, d, G)
    qt = bits_to_dev(q, (B, Hq, d))
    kt = bits_to_dev(kc, (B, Lmax, Hkv, d))
    vt = bits_to_dev(vc, (B, Lmax, Hkv, d))
    cl = torch.tensor(lens, dtype=torch.int32, device=dev())
    qp = torch.tensor(lens, dtype=torch.int32, device=dev())
    cnt = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev())
    o = W.decode(qt, kt, vt, cl, qp, cut, G, counters=cnt, out=out, num_splits=3)
    torch.cuda.synchronize()
    got = bf16_to_np(o)
    dim_cut = O.dim_cutoffs_grouped(np.array(cut), G)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(got[b], np.zeros((Hq, d))), b
        else:
            sl = slice(b * Lmax, b * Lmax + Lmax)
            ref = O.decode(to_f64(q[b]), to_f64(kc[sl]), to_f64(vc[sl]), L, L, dim_cut)
            compare(got[b], ref, "decode b=%d L=%d" % (b, L))
    exp = _expected(lens, lens, d, G, cut, Hkv)
    assert np.array_equal(cnt.cpu().numpy(), exp)


def test_decode_strided_views():
    """K and V as views into one interleaved cache [B, Lmax, 2, Hkv, d] (the
    layout of frameworks that keep K and V of a token together), q as a view
    into a wider tensor and o written into a wider buffer: bit-identical to
    the contiguous call, and the buffer outside o untouched."""
    B, Lmax, Hq, Hkv, d, G, theta = 3, 700, 16, 4, 128, 16, 300.0
    lens = [700, 513, 64]
    q = synth.normal_bits(41, 0, B, (Hq, d))
    kc = synth.normal_bits(41, 1, B * Lmax, (Hkv, d))
    vc = synth.normal_bits(41, 2, B * Lmax, (Hkv, d))
    cut = W.group_cutoffs(theta, d, G)
    qt = bits_to_dev(q, (B, Hq, d))
    kt = bits_to_dev(kc, (B, Lmax, Hkv, d))
    vt = bits_to_dev(vc, (B, Lmax, Hkv, d))
    cl = torch.tensor(lens, dtype=torch.int32, device=dev())
    qp = torch.tensor(lens, dtype=torch.int32, device=dev())
    o1 = W.decode(qt, kt, vt, cl, qp, cut, G, num_splits=4)
    kv = torch.stack([kt, vt], dim=2)                     # [B, Lmax, 2, Hkv, d]
    qwide = torch.zeros((B, Hq + 3, d), dtype=torch.bfloat16, device=dev())
    qwide[:, 1:1 + Hq] = qt
    big = torch.zeros((B, Hq + 5, d), dtype=torch.bfloat16, device=dev())
    o2 = W.decode(qwide[:, 1:1 + Hq], kv[:, :, 0], kv[:, :, 1], cl, qp, cut, G, num_splits=4,
                  out=big[:, 2:2 + Hq])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.count_nonzero(big[:, :2]) == 0 and torch.count_nonzero(big[:, 2 + Hq:]) == 0


# B, Lmax, Hq, Hkv, d, G, theta, cache lengths, splits
WIDE_GQA = [
    (2, 900, 32, 1, 128, 16, 1e3, [900, 451], 0),      # 32 query heads on one kv head: two head sets
    (1, 1500, 40, 2, 64, 32, 300.0, [1500], 3),         # 20 per kv head: sets of 16 and 4
    (2, 700, 48, 2, 128, 2, 1e4, [700, 1], 0),          # 24 per kv head, exact rule
    (1, 600, 64, 1, 128, 16, 1e3, [600], 0),            # 64 per kv head: two passes of 32
    (1, 700, 80, 2, 64, 32, 1e4, [700], 2),             # 40 per kv head: passes of 32 and 8
    (2, 500, 17, 1, 128, 4, 300.0, [500, 33], 0),       # 17: the second set holds one head
]


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,d,G,theta,lens,splits", WIDE_GQA)
def test_decode_wide_gqa(B, Lmax, Hq, Hkv, d, G, theta, lens, splits):
    """More than 16 query heads per kv head (MQA-style): up to 32 heads share
    one pass over the cache as two MFMA head sets, more run in passes of 32;
    every head against the oracle and the tile counters counted once per
    (sequence, kv head, key block)."""
    say("decode wide GQA: B=%d Lmax=%d Hq=%d Hkv=%d d=%d G=%d lens=%s" % (B, Lmax, Hq, Hkv, d, G, lens))
    q = synth.normal_bits(47, 0, B, (Hq, d))
    kc = synth.normal_bits(47, 1, B * Lmax, (Hkv, d))
    vc = synth.normal_bits(47, 2, B * Lmax, (Hkv, d))
    cut = W.group_cutoffs(theta, d, G)
    qt = bits_to_dev(q, (B, Hq, d))
    kt = bits_to_dev(kc, (B, Lmax, Hkv, d))
    vt = bits_to_dev(vc, (B, Lmax, Hkv, d))
    cl = torch.tensor(lens, dtype=torch.int32, device=dev())
    qp = torch.tensor(lens, dtype=torch.int32, device=dev())
    cnt = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    o = W.decode(qt, kt, vt, cl, qp, cut, G, counters=cnt, num_splits=splits)
    torch.cuda.synchronize()
    got = bf16_to_np(o)
    dim_cut = O.dim_cutoffs_exact(theta, d) if G == 2 else O.dim_cutoffs_grouped(np.array(cut), G)
    for b in range(B):
        sl = slice(b * Lmax, (b + 1) * Lmax)
        ref = O.decode(to_f64(q[b]), to_f64(kc[sl]), to_f64(vc[sl]), lens[b], lens[b], dim_cut)
        compare(got[b], ref, "decode wide GQA b=%d" % b)
    assert np.array_equal(cnt.cpu().numpy(), _expected(lens, lens, d, G, cut, Hkv))


def test_decode_cache_past_2gib():
    """A cache longer than one 32-bit buffer resource could span: one
    sequence of 3 x 2^19 keys (1.5 M) whose token stride is 2 KB (the cache
    holds 8 kv heads; the last one is used through a strided view), so its
    keys reach 3 GiB past the sequence start.  Every 32-key block is read
    through its own resources.  Against the oracle, counters bit-exact."""
    L, Hq, Hkv, Hall, d, G, theta = 3 << 19, 4, 1, 8, 128, 16, 1e6
    say("decode past 2 GiB: L=%d token stride %d bytes, span %.2f GiB" % (L, Hall * d * 2, L * Hall * d * 2 / 2 ** 30))
    q = synth.normal_bits(83, 0, 1, (Hq, d))
    kc = synth.normal_bits(83, 1, L, (Hkv, d))
    vc = synth.normal_bits(83, 2, L, (Hkv, d))
    kbig = torch.zeros((1, L, Hall, d), dtype=torch.bfloat16, device=dev())
    vbig = torch.zeros((1, L, Hall, d), dtype=torch.bfloat16, device=dev())
    kbig[:, :, Hall - Hkv:] = bits_to_dev(kc, (1, L, Hkv, d))
    vbig[:, :, Hall - Hkv:] = bits_to_dev(vc, (1, L, Hkv, d))
    cut = W.group_cutoffs(theta, d, G)
    qt = bits_to_dev(q, (1, Hq, d))
    cl = torch.tensor([L], dtype=torch.int32, device=dev())
    qp = torch.tensor([L], dtype=torch.int32, device=dev())
    cnt = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    o = W.decode(qt, kbig[:, :, Hall - Hkv:], vbig[:, :, Hall - Hkv:], cl, qp, cut, G, counters=cnt)
    torch.cuda.synchronize()
    got = bf16_to_np(o)[0]
    del kbig, vbig
    ref = O.decode(to_f64(q[0]), to_f64(kc), to_f64(vc), L, L, O.dim_cutoffs_grouped(np.array(cut), G))
    compare(got, ref, "decode L=1.5M (3 GiB span)")
    assert np.array_equal(cnt.cpu().numpy(), _expected([L], [L], d, G, cut, Hkv))
