#!/usr/bin/env python3
"""Benchmark of the WavePrune hot path on one MI355X; prints one JSON line.

A step is one pass of the whole path over resident synthetic inputs:
  RoPE of Q and K (32K prefill) -> WavePrune prefill (32K, 32/8 heads,
  d_h 128, theta 1e6, G 16) -> RoPE of the 16 decode queries -> WavePrune
  decode (16 sequences x 32K cached tokens, 32/8 heads).
The in-house dense baseline (same kernels, every group full) is timed the
same way right after, for the speedups.  Kernel times come from HIP events
recorded on the stream the library launches on.  The decode figures (and its
roofline) come from the decode timed on its own as the pages time it (10
warmups, median of 50 back-to-back launches, two cache copies alternating);
the decode time inside the step, right after the prefill, is reported too.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("prefill dense-equiv TFLOPS + decode KV GB/s at 32K, d_h=128; "
          "speedup vs own dense")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# work accounting (per launch)
# ---------------------------------------------------------------------------
def prefill_flops(n, Hq, B, d_h, G, cut):
    """Dense-equivalent, algorithmic (per causal pair: 2*G per kept group +
    2*d_h for P.V) and executed (per visited 32x32 tile: 2*32*32*G per
    non-skipped group + 2*32*32*d_h) FLOPs."""
    import rope_positional_encoding_amd as W
    dense = 4.0 * d_h * n * (n + 1) / 2.0
    alg = 2.0 * d_h * n * (n + 1) / 2.0
    for D in cut:
        m = min(int(D), n - 1)
        # causal pairs with distance 0..m: sum_{t=0..m} (n - t)
        alg += 2.0 * G * ((m + 1) * n - m * (m + 1) / 2.0)
    cnt = W.prefill_tile_counts(n, d_h, G, cut)
    ng = d_h // G
    BM, BN = W.prefill_tiling(d_h, G)
    tile = 2.0 * BM * BN
    visited = cnt[3 * ng]
    exe = visited * tile * d_h
    for g in range(ng):
        exe += (cnt[3 * g + 1] + cnt[3 * g + 2]) * tile * G
    k = B * Hq
    return dense * k, alg * k, exe * k


def backward_flops(dense_fwd_flops, alg_fwd_flops):
    """Dense-equivalent and algorithmic FLOPs of the prefill backward from the
    forward's: five d_h-long products per causal pair (S, dP, dV, dK, dQ) =
    2.5x the dense forward; algorithmically dP and dV cover every dim while
    S, dK and dQ cover the kept groups only, i.e. 2 x the forward's P.V part
    (half its dense work) + 3 x its kept-group QK part."""
    pv = dense_fwd_flops / 2.0
    return 2.5 * dense_fwd_flops, 2.0 * pv + 3.0 * (alg_fwd_flops - pv)


def decode_bytes(L, q_pos, Hkv, Hq, B, d_h, G, cut):
    """Dense KV bytes, algorithmic bytes (kept K groups + all V + q/o) and
    the bytes of the K/V reads the kernel issues (per 32-key block)."""
    import rope_positional_encoding_amd as W
    dense = 2.0 * 2 * L * d_h
    kept_k = 0.0
    for D in cut:
        # keys j with q_pos - j <= D, j in [0, L)
        lo = max(0, q_pos - int(D))
        kept_k += 2.0 * G * max(0, L - lo)
    alg = kept_k + 2.0 * L * d_h
    cnt = W.decode_tile_counts(q_pos, L, d_h, G, cut)
    ng = d_h // G
    BN = W.decode_tiling(d_h, G)
    issued = 0.0
    for g in range(ng):
        issued += (cnt[3 * g + 1] + cnt[3 * g + 2]) * BN * 2.0 * G
    issued += 2.0 * L * d_h
    k = B * Hkv
    qo = 2.0 * 2 * B * Hq * d_h
    return dense * k, alg * k + qo, issued * k + qo


# ---------------------------------------------------------------------------
KERNEL_SOURCES = {
    "prefill": ["rope_positional_encoding_amd/csrc/prefill.hip", "rope_positional_encoding_amd/csrc/wp_internal.h",
                "rope_positional_encoding_amd/build.py"],
    "decode": ["rope_positional_encoding_amd/csrc/decode.hip", "rope_positional_encoding_amd/csrc/wp_internal.h",
               "rope_positional_encoding_amd/build.py"],
    "decode_kcache": ["rope_positional_encoding_amd/csrc/decode.hip",
                      "rope_positional_encoding_amd/csrc/wp_internal.h", "rope_positional_encoding_amd/build.py"],
}
for _srcs in KERNEL_SOURCES.values():
    _srcs.append("rope_positional_encoding_amd/csrc/wp_device.h")


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    calibration) from profiles/traffic.txt, only if it was measured on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and not line.startswith("#") and f[0] == kernel:
            if f[1] != source_hash(kernel):
                return None
            return float(f[2]) + float(f[3])
    return None


# ---------------------------------------------------------------------------
def _oracle_threads():
    """Host threads for the oracle: the CPUs this process may run on, at
    most 16 (a host share of 16 threads per GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _timed_rows(fn, items, threads, budget_s=None):
    """Run fn(item) over items on `threads` host threads (one BLAS thread
    each), stopping at budget_s seconds if given; returns (done_items,
    seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    done = []
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        if threads <= 1:
            for it in items:
                fn(it)
                done.append(it)
                if budget_s is not None and time.perf_counter() - t0 > budget_s and len(done) >= 4:
                    break
        else:
            with ThreadPoolExecutor(threads) as ex:
                pos = 0
                while pos < len(items):
                    batch = items[pos:pos + 4 * threads]
                    list(ex.map(fn, batch))
                    done.extend(batch)
                    pos += len(batch)
                    if budget_s is not None and time.perf_counter() - t0 > budget_s:
                        break
    return done, time.perf_counter() - t0


def _f64(t):
    import numpy as np
    return t.float().cpu().numpy().astype(np.float64)


def oracle_prefill_rate(qr, kr, v, rows, dim_cut, threads, budget_s=None):
    """The oracle (as it stands) on the given query rows of batch 0 of a
    prefill, one row per task; returns (rows done, seconds, dense-equivalent
    FLOPs of those rows)."""
    import numpy as np
    import torch
    import oracle as O
    Hq, d = qr.shape[2], qr.shape[3]
    rows = [int(r) for r in rows]
    ridx = torch.tensor(rows, device=qr.device)
    q64 = _f64(qr[0, ridx])
    k64, v64 = _f64(kr[0]), _f64(v[0])
    where = {r: i for i, r in enumerate(rows)}

    def one(i):
        j = where[i]
        O.prefill(q64[j:j + 1], k64, v64, dim_cut, rows=[i], q_is_rows=True)

    done, dt = _timed_rows(one, rows, threads, budget_s)
    flops = sum(4.0 * d * Hq * (i + 1) for i in done)
    return np.array(done), dt, flops


def cpu_baseline(qr, kr, v, n, Hq, d_h, G, theta, seconds, seed=11, max_rows=4096):
    """The CPU oracle (float64 numpy, as it stands) on seeded uniform query
    rows of the 32K prefill (the rotated inputs the GPU consumed), on every
    host CPU available (one row per thread), and on one thread for
    comparison; scaled to dense-equivalent TFLOP/s."""
    import numpy as np
    import oracle as O

    rng = np.random.default_rng(seed)
    rows = rng.integers(0, n, size=max_rows)
    dc = O.dim_cutoffs_grouped(O.group_cutoffs(theta, d_h, G), G)
    threads = _oracle_threads()
    done, dt, flops = oracle_prefill_rate(qr, kr, v, rows, dc, threads, seconds)
    done1, dt1, flops1 = oracle_prefill_rate(qr, kr, v, rows[:64], dc, 1, seconds / 3)
    # labelled extrapolation to the whole prefill: the oracle's cost per row
    # grows with the row's causal length, so scale by sum(i + 1) over all rows
    # / over the sampled rows
    scale = (n * (n + 1) / 2.0) / float(np.sum(done + 1))
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s (prefill, dense-equivalent)",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d seeded uniform query rows x %d heads of the 32K prefill (grouped rule, float64 "
                  "numpy), one row per host thread on %d threads, %.1f s" % (len(done), Hq, threads, dt),
        "extrapolated_full_prefill_s": round(dt * scale, 1),
        "single_thread": {"value": flops1 / dt1 / 1e12, "cores": 1,
                          "sample": "%d of the same rows on one thread, %.1f s" % (len(done1), dt1)},
        "host_cpus_available": len(os.sched_getaffinity(0)),
    }


# The other prefill workloads (the headline is the 32K G = 16 prefill and the
# 16 x 32K decode): name -> (B, n, Hq, Hkv, d_h, G, theta, pos_scale, fp32 Q/K,
# per-channel std, oracle rows (0 = all), warmups, timed launches)
PREFILL_CONFIGS = {
    "tiny256": (1, 256, 1, 1, 64, 16, 1e4, 1.0, True, False, 0, 3, 10),
    "prefill4k": (1, 4096, 32, 8, 128, 16, 1e6, 1.0, False, True, 0, 3, 10),
    "prefill32k_g32": (1, 32768, 32, 8, 128, 32, 1e6, 1.0, False, False, 256, 3, 10),
    "prefill128k_s4": (1, 131072, 64, 8, 128, 16, 1e6, 4.0, False, False, 128, 1, 3),
}


# evaluation variants timed next to the default kernel of a workload
PREFILL_VARIANTS = {"prefill32k_g32": ("mfma16x16x32",)}


def _time_launches(fn, warmup, reps):
    """warmup calls, then reps calls each bracketed by events on the launch
    stream; returns the times in ms."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def bench_prefill_config(W, name, gen, with_oracle, extra_flags=()):
    """One prefill workload: RoPE of the raw Q and K, then the WavePrune
    prefill and the dense baseline, each timed as the pages time prefill
    (warmups, then the median of the timed launches).  With with_oracle, the
    oracle is timed on the workload's rows (all, or the sampled rows with the
    labelled extrapolation to the whole prefill) on every host thread."""
    import numpy as np
    import torch
    from rope_positional_encoding_amd import synth
    B, n, Hq, Hkv, d, G, theta, s, fp32, chstd, orows, warm, reps = PREFILL_CONFIGS[name]
    log("bench: %s" % name)
    dev = torch.device("cuda:0")
    dt_in = torch.float32 if fp32 else torch.bfloat16

    def randn(shape, tid):
        x = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
        if chstd:
            x *= torch.from_numpy(synth.channel_std(2, tid, d)).to(dev)
        return x.to(dt_in)

    q_raw = randn((B, n, Hq, d), synth.TID_Q)
    k_raw = randn((B, n, Hkv, d), synth.TID_K)
    v = randn((B, n, Hkv, d), synth.TID_V).to(torch.bfloat16)
    qr = W.rope_apply(q_raw, theta, s)
    kr = W.rope_apply(k_raw, theta, s)
    o = torch.empty_like(qr)
    cut = W.group_cutoffs(theta, d, G, s)
    rope_ms = statistics.median(_time_launches(
        lambda: (W.rope_apply(q_raw, theta, s, out=qr), W.rope_apply(k_raw, theta, s, out=kr)), 2, 5))
    wp = _time_launches(lambda: W.prefill(qr, kr, v, cut, G, out=o), warm, reps)
    dn = _time_launches(lambda: W.prefill(qr, kr, v, None, G, dense=True, out=o), warm, reps)
    dense_f, alg_f, exe_f = prefill_flops(n, Hq, B, d, G, cut)
    med, med_d = statistics.median(wp), statistics.median(dn)
    avg = sum(wp) / len(wp)
    ach = alg_f / (avg * 1e-3) / 1e12
    res = {"shape": {"B": B, "n": n, "Hq": Hq, "Hkv": Hkv, "d_h": d, "theta": theta, "pos_scale": s, "G": G,
                     "inputs": "fp32 Q/K" if fp32 else ("bf16, per-channel std U[0.5,2]" if chstd else "bf16")},
           "protocol": "%d warmups, median of %d launches" % (warm, reps),
           "ms_median": round(med, 4), "ms_min": round(min(wp), 4), "ms_max": round(max(wp), 4),
           "dense_equiv_tflops": round(dense_f / (med * 1e-3) / 1e12, 2),
           "algorithmic_tflops": round(alg_f / (med * 1e-3) / 1e12, 2),
           "executed_tflops": round(exe_f / (med * 1e-3) / 1e12, 2),
           "algorithmic_fraction_of_dense": round(alg_f / dense_f, 4),
           "dense_ms_median": round(med_d, 4),
           "dense_tflops": round(dense_f / (med_d * 1e-3) / 1e12, 2),
           "dense_frac_of_peak": round(dense_f / (med_d * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "speedup_vs_dense": round(med_d / med, 4),
           "rope_q_k_ms": round(rope_ms, 4),
           "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4), "avg_ms": round(avg, 4),
                        "kernel": "prefill_kernel<%d,%d>" % (d, G)}}
    for fl in extra_flags:
        # evaluation variants of the same prefill (same result, other tiling)
        vt = _time_launches(lambda: W.prefill(qr, kr, v, cut, G, out=o, variant=fl), warm, reps)
        vm, va = statistics.median(vt), sum(vt) / len(vt)
        vd = _time_launches(lambda: W.prefill(qr, kr, v, None, G, dense=True, out=o, variant=fl), warm, reps)
        res["variant_" + fl] = {"ms_median": round(vm, 4), "dense_ms_median": round(statistics.median(vd), 4),
                                "speedup_vs_dense": round(statistics.median(vd) / vm, 4),
                                "algorithmic_tflops": round(alg_f / (vm * 1e-3) / 1e12, 2),
                                "frac": round(alg_f / (va * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                "time_vs_default": round(vm / med, 4)}
    cpu = None
    if with_oracle:
        import oracle as O
        dc = O.dim_cutoffs_grouped(np.array(cut), G)
        if orows == 0:
            rows = np.arange(n)
        else:
            rows = synth.sample_rows(n, orows, 7, [c + e for c in cut for e in (0, 1)])
        threads = _oracle_threads()
        done, dt, flops = oracle_prefill_rate(qr, kr, v, rows, dc, threads)
        cpu = {"rows": "all %d" % n if orows == 0 else "%d sampled rows" % len(done), "seconds": round(dt, 2),
               "threads": threads, "dense_equiv_tflops": flops / dt / 1e12 * B}
        if orows:
            scale = (n * (n + 1) / 2.0) / float(np.sum(done + 1))
            cpu["extrapolated_full_prefill_s"] = round(dt * scale * B, 1)
            cpu["extrapolation"] = "x sum(i+1) over all rows / over the sampled rows"
    del q_raw, k_raw, v, qr, kr, o
    torch.cuda.empty_cache()
    return res, cpu


def oracle_decode_rate(dq, kc, vc, L, q_pos, cut, G, threads):
    """The oracle on every sequence of a decode (all cached keys), one
    sequence per host thread; returns (seconds, dense KV bytes)."""
    import numpy as np
    import oracle as O
    dc = O.dim_cutoffs_grouped(np.array(cut), G)
    B = dq.shape[0]
    q64 = _f64(dq)
    ks = [_f64(kc[b, :L]) for b in range(B)]
    vs = [_f64(vc[b, :L]) for b in range(B)]
    _, dt = _timed_rows(lambda b: O.decode(q64[b], ks[b], vs[b], q_pos, L, dc), list(range(B)), threads)
    return dt, 2.0 * 2 * B * L * kc.shape[2] * kc.shape[3]


def bench_backward(W, q, k, v, cut, G, n, Hq, d, dense_fwd_flops, alg_fwd_flops):
    """wp_prefill_backward at the prefill shape: 1 warmup, median of 3, for
    the WavePrune table and the dense baseline.  Dense-equivalent work: five
    d_h-long products per causal pair (S, dP, dV, dK, dQ) = 2.5x the forward.
    Algorithmic work: dP and dV over all d_h dims, S, dK and dQ over the kept
    groups only, i.e. 2 x (the forward's P.V part) + 3 x (its kept-group QK
    part); the roofline fraction is taken on it, as for the forward."""
    import torch
    log("bench: prefill backward")
    o, lse = W.prefill(q, k, v, cut, G, return_lse=True)
    od, lsed = W.prefill(q, k, v, None, G, dense=True, return_lse=True)
    g = torch.randn(q.shape, device=q.device, dtype=torch.float32).to(torch.bfloat16)
    ws = torch.empty(W.lib().wp_prefill_backward_workspace_size(1, n, Hq), dtype=torch.uint8, device=q.device)
    res = {}
    for dense in (False, True):
        oo, ll = (od, lsed) if dense else (o, lse)
        W.prefill_backward(q, k, v, oo, g, ll, None if dense else cut, G, dense=dense, workspace=ws)
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            W.prefill_backward(q, k, v, oo, g, ll, None if dense else cut, G, dense=dense, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res["dense" if dense else "wp"] = statistics.median(ts)
    bwd_flops, bwd_alg = backward_flops(dense_fwd_flops, alg_fwd_flops)
    alg_tflops = bwd_alg / (res["wp"] * 1e-3) / 1e12
    return {"ms_median": round(res["wp"], 3), "dense_ms_median": round(res["dense"], 3),
            "dense_equiv_tflops": round(bwd_flops / (res["wp"] * 1e-3) / 1e12, 2),
            "algorithmic_tflops": round(alg_tflops, 2),
            "algorithmic_fraction_of_dense": round(bwd_alg / bwd_flops, 4),
            "frac_of_peak": round(alg_tflops / PEAK_BF16_TFLOPS, 4),
            "dense_tflops": round(bwd_flops / (res["dense"] * 1e-3) / 1e12, 2),
            "dense_frac_of_peak": round(bwd_flops / (res["dense"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "speedup_vs_dense": round(res["dense"] / res["wp"], 4)}


def bench_kcache(W, q, kcs, vcs, cl, qp, cut, G, ws, od, dec_alg, full_ms):
    """The same decode with K read from the group-major compact store (group
    g keeps only its last D'_g + 1 keys), one store per cache copy, timed as
    time_decode."""
    import torch
    log("bench: decode from the compact K store")
    B, L, Hkv, d = kcs[0].shape
    stores = []
    for kc in kcs:
        st = W.kcache_empty(B, Hkv, L, d, G, cut, device=kc.device)
        W.kcache_append(kc, torch.zeros(B, dtype=torch.int32, device=kc.device), st, L, cut, G)
        stores.append(st)
    store = stores[0]
    ms = time_decode(W, q, stores, vcs, cl, qp, cut, G, ws, od, compact=True)
    med = statistics.median(ms)
    k_full = float(kcs[0].numel() * 2)
    k_store = float(store.numel() * 2)
    avg = sum(ms) / len(ms)
    ach = dec_alg / (avg * 1e-3) / 1e9
    return {"ms_median": round(med, 4), "ms_min": round(min(ms), 4),
            "algorithmic_gbs": round(dec_alg / (med * 1e-3) / 1e9, 1),
            "k_store_bytes": k_store, "k_cache_bytes": k_full,
            "k_capacity_fraction": round(k_store / k_full, 4),
            "kv_capacity_fraction": round((k_store + k_full) / (2 * k_full), 4),
            "time_vs_full_cache_decode": round(med / full_ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode_kcache"),
                         "algorithmic_bytes": dec_alg,
                         "kernel": "decode_split_kernel<128,16,compact> + decode_merge_kernel<128>",
                         "avg_ms": round(avg, 4)}}


def time_decode(W, dq, kcs, vcs, cl, qp, cut, G, ws, od, dense=False, warmup=10, reps=50, compact=False):
    """Decode timed on its own, as the pages time it: 10 warmups, then 50
    launches with events on the launch stream and no host sync in between
    (one untimed launch is queued first, so the host stays ahead of the GPU),
    alternating between two copies of the KV cache.  Returns the times (ms)."""
    import torch

    def call(i):
        if compact:
            W.decode_kcache(dq, kcs[i & 1], vcs[i & 1], cl, qp, cut, G, workspace=ws, out=od)
        else:
            W.decode(dq, kcs[i & 1], vcs[i & 1], cl, qp, None if dense else cut, G, dense=dense,
                     workspace=ws, out=od)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    call(1)
    s = torch.cuda.current_stream()
    pairs = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        call(i)
        e1.record(s)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def bench_exact(W, qr, kr, v, dq, kcs, vcs, cl, qp, ws, od, theta, n, Hq, Hkv, d, Bd, L, q_pos,
                grouped_prefill_ms, grouped_decode_ms, grouped_backward_ms=None):
    """The exact per-channel rule (G = 2: every channel its own cutoff) on the
    same prefill and decode workloads: the prefill 2 warmups, then 5 launches
    timed with events on the launch stream (the backward, when the grouped
    one was timed, 2 warmups and 3 launches); the decode as time_decode over
    the two cache copies kcs, vcs."""
    import torch
    log("bench: exact per-channel rule (G = 2)")
    G2 = 2
    cut2 = W.group_cutoffs(theta, d, G2)
    o2 = torch.empty_like(qr)

    def timed(fn, reps):
        fn()
        fn()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        pairs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in pairs]

    pm = timed(lambda: W.prefill(qr, kr, v, cut2, G2, out=o2), 5)
    bm = None
    if grouped_backward_ms is not None:
        _, lse2 = W.prefill(qr, kr, v, cut2, G2, out=o2, return_lse=True)
        g = torch.randn(qr.shape, device=qr.device, dtype=torch.float32).to(torch.bfloat16)
        bm = timed(lambda: W.prefill_backward(qr, kr, v, o2, g, lse2, cut2, G2), 3)
    dm = time_decode(W, dq, kcs, vcs, cl, qp, cut2, G2, ws, od)
    dense_f, alg_f, _ = prefill_flops(n, Hq, 1, d, G2, cut2)
    _, dec_alg, _ = decode_bytes(L, q_pos, Hkv, Hq, Bd, d, G2, cut2)
    p_med, d_med = statistics.median(pm), statistics.median(dm)
    p_avg, d_avg = sum(pm) / len(pm), sum(dm) / len(dm)
    ach = alg_f / (p_avg * 1e-3) / 1e12
    ach_d = dec_alg / (d_avg * 1e-3) / 1e9
    out = {"G": G2,
            "prefill": {"ms_median": round(p_med, 4),
                        "dense_equiv_tflops": round(dense_f / (p_med * 1e-3) / 1e12, 2),
                        "algorithmic_tflops": round(alg_f / (p_med * 1e-3) / 1e12, 2),
                        "algorithmic_fraction_of_dense": round(alg_f / dense_f, 4),
                        "time_vs_grouped": round(p_med / grouped_prefill_ms, 4),
                        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                                     "traffic": None, "kernel": "prefill_kernel<128,2>",
                                     "avg_ms": round(p_avg, 4)}},
            "decode": {"ms_median": round(d_med, 4),
                       "algorithmic_gbs": round(dec_alg / (d_med * 1e-3) / 1e9, 1),
                       "time_vs_grouped": round(d_med / grouped_decode_ms, 4),
                       "roofline": {"bound": "hbm", "achieved": round(ach_d, 1), "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": round(ach_d / PEAK_HBM_GBS, 4), "traffic": None,
                                    "algorithmic_bytes": dec_alg,
                                    "kernel": "decode_split_kernel<128,2> + decode_merge_kernel<128>",
                                    "avg_ms": round(d_avg, 4)}}}
    if bm is not None:
        b_med = statistics.median(bm)
        out["prefill_backward"] = {"ms_median": round(b_med, 3),
                                   "time_vs_grouped": round(b_med / grouped_backward_ms, 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-kcache", action="store_true", help="skip the compact K store decode line")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill backward line")
    ap.add_argument("--no-exact", action="store_true", help="skip the exact per-channel rule (G = 2) line")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other prefill workloads (tiny256, prefill4k, prefill32k_g32, prefill128k_s4)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (3 launches): a kernel of known "
                         "traffic for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the path needs no "
              "collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import rope_positional_encoding_amd as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # prefill32k_g16 and decode32k shapes
    n, Hq, Hkv, d, G, theta = 32768, 32, 8, 128, 16, 1e6
    Bd, L, q_pos = 16, 32768, 32768
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261203)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("bench: allocating inputs")
    q_raw = randn(1, n, Hq, d)
    k_raw = randn(1, n, Hkv, d)
    v = randn(1, n, Hkv, d)
    qr = torch.empty_like(q_raw)
    kr = torch.empty_like(k_raw)
    o = torch.empty_like(q_raw)
    dq_raw = randn(Bd, 1, Hq, d)
    dqr = torch.empty_like(dq_raw)
    kc = W.rope_apply(randn(Bd, L, Hkv, d), theta)     # the cache holds rotated keys
    vc = randn(Bd, L, Hkv, d)
    kcs, vcs = (kc, kc.clone()), (vc, vc.clone())      # two cache copies for the decode loop
    od = torch.empty(Bd, Hq, d, dtype=torch.bfloat16, device=dev)
    cl = torch.full((Bd,), L, dtype=torch.int32, device=dev)
    qp = torch.full((Bd,), q_pos, dtype=torch.int32, device=dev)
    qp64 = torch.full((Bd,), q_pos, dtype=torch.int64, device=dev)
    ws = torch.empty(W.decode_workspace_size(Bd, L, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    cut = W.group_cutoffs(theta, d, G)
    torch.cuda.synchronize()

    names = ["rope_q", "rope_k", "prefill", "rope_dq", "decode"]

    def step(ev, dense=False):
        s = torch.cuda.current_stream()
        e = ev
        e[0].record(s)
        W.rope_apply(q_raw, theta, out=qr)
        e[1].record(s)
        W.rope_apply(k_raw, theta, out=kr)
        e[2].record(s)
        W.prefill(qr, kr, v, None if dense else cut, G, dense=dense, out=o)
        e[3].record(s)
        W.rope_apply(dq_raw, theta, pos_start=qp64, out=dqr)
        e[4].record(s)
        W.decode(dqr[:, 0], kc, vc, cl, qp, None if dense else cut, G, dense=dense,
                 workspace=ws, out=od)
        e[5].record(s)

    def run(dense):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        warm = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for _ in range(args.warmup):
            step(warm, dense)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(evs[k], dense)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {nm: [evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(args.steps)]
               for i, nm in enumerate(names)}
        total = sum(evs[k][0].elapsed_time(evs[k][5]) for k in range(args.steps))
        return per, total / args.steps, wall

    log("bench: WavePrune steps")
    per, ms_step, wall = run(False)
    log("bench: dense baseline steps")
    per_d, ms_step_d, _ = (None, None, None) if args.no_dense else run(True)

    med = {k: statistics.median(v_) for k, v_ in per.items()}
    avg = {k: sum(v_) / len(v_) for k, v_ in per.items()}
    # decode on its own (inside the step it follows the prefill, whose dirty
    # output lines are written back to HBM during the decode)
    log("bench: decode on its own")
    dec_ms = time_decode(W, dqr[:, 0], kcs, vcs, cl, qp, cut, G, ws, od)
    dec_ms_d = None if args.no_dense else time_decode(W, dqr[:, 0], kcs, vcs, cl, qp, cut, G, ws, od,
                                                      dense=True)
    dmed, davg = statistics.median(dec_ms), sum(dec_ms) / len(dec_ms)
    dense_f, alg_f, exe_f = prefill_flops(n, Hq, 1, d, G, cut)
    kv_dense, dec_alg, dec_issued = decode_bytes(L, q_pos, Hkv, Hq, Bd, d, G, cut)
    rope_bytes = 2 * 2.0 * (q_raw.numel() + k_raw.numel())
    prefill_bytes = 2.0 * (2 * q_raw.numel() + 2 * k_raw.numel())   # read q, k, v; write o

    out = {
        "metric": METRIC,
        "value": round(dense_f / (med["prefill"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill32k_g16 + decode32k",
                   "prefill": {"B": 1, "n": n, "Hq": Hq, "Hkv": Hkv, "d_h": d, "theta": theta, "G": G},
                   "decode": {"B": Bd, "cache_len": L, "q_pos": q_pos, "Hq": Hq, "Hkv": Hkv,
                              "d_h": d, "theta": theta, "G": G}},
        "prefill": {
            "ms_median": round(med["prefill"], 4), "ms_min": round(min(per["prefill"]), 4),
            "ms_max": round(max(per["prefill"]), 4),
            "dense_equiv_tflops": round(dense_f / (med["prefill"] * 1e-3) / 1e12, 2),
            "algorithmic_tflops": round(alg_f / (med["prefill"] * 1e-3) / 1e12, 2),
            "executed_tflops": round(exe_f / (med["prefill"] * 1e-3) / 1e12, 2),
            "algorithmic_fraction_of_dense": round(alg_f / dense_f, 4),
            "executed_fraction_of_dense": round(exe_f / dense_f, 4),
        },
        "decode": {
            "protocol": "10 warmups, median of 50 back-to-back launches, two cache copies alternating",
            "ms_median": round(dmed, 4), "ms_min": round(min(dec_ms), 4), "ms_max": round(max(dec_ms), 4),
            "kv_gbs_dense_equiv": round(kv_dense / (dmed * 1e-3) / 1e9, 1),
            "algorithmic_gbs": round(dec_alg / (dmed * 1e-3) / 1e9, 1),
            "issued_gbs": round(dec_issued / (dmed * 1e-3) / 1e9, 1),
            "algorithmic_fraction_of_dense": round(dec_alg / kv_dense, 4),
            "in_step_ms_median": round(med["decode"], 4),
            "in_step_algorithmic_gbs": round(dec_alg / (med["decode"] * 1e-3) / 1e9, 1),
        },
        "rope": {"ms_q": round(med["rope_q"], 4), "ms_k": round(med["rope_k"], 4),
                 "gbs": round(rope_bytes / ((med["rope_q"] + med["rope_k"]) * 1e-3) / 1e9, 1)},
    }
    if per_d is not None:
        med_d = {k: statistics.median(v_) for k, v_ in per_d.items()}
        out["prefill"]["dense_ms_median"] = round(med_d["prefill"], 4)
        out["prefill"]["dense_tflops"] = round(dense_f / (med_d["prefill"] * 1e-3) / 1e12, 2)
        # the dense baseline executes every FLOP it is credited with: its own fraction of the MFMA peak
        out["prefill"]["dense_frac_of_peak"] = round(dense_f / (med_d["prefill"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        out["prefill"]["speedup_vs_dense"] = round(med_d["prefill"] / med["prefill"], 4)
        dmed_d = statistics.median(dec_ms_d)
        out["decode"]["dense_ms_median"] = round(dmed_d, 4)
        out["decode"]["dense_kv_gbs"] = round(kv_dense / (dmed_d * 1e-3) / 1e9, 1)
        out["decode"]["dense_frac_of_peak"] = round(kv_dense / (dmed_d * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        out["decode"]["speedup_vs_dense"] = round(dmed_d / dmed, 4)
        out["decode"]["in_step_dense_ms_median"] = round(med_d["decode"], 4)
        out["decode"]["in_step_speedup_vs_dense"] = round(med_d["decode"] / med["decode"], 4)
    # roofline of the dominant kernel (prefill): algorithmic FLOPs per launch
    # over the average launch duration measured with events on its stream
    ach = alg_f / (avg["prefill"] * 1e-3) / 1e12
    out["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                       "traffic": measured_traffic("prefill"), "algorithmic_bytes": prefill_bytes,
                       "kernel": "prefill_kernel<128,16>", "avg_ms": round(avg["prefill"], 4)}
    ach_d = dec_alg / (davg * 1e-3) / 1e9
    out["roofline_decode"] = {"bound": "hbm", "achieved": round(ach_d, 1), "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": round(ach_d / PEAK_HBM_GBS, 4),
                              "traffic": measured_traffic("decode"), "algorithmic_bytes": dec_alg,
                              "kernel": "decode_split_kernel<128,16> + decode_merge_kernel<128>",
                              "avg_ms": round(davg, 4)}
    bwd_ms = None
    if not args.no_backward:
        out["prefill_backward"] = bench_backward(W, qr, kr, v, cut, G, n, Hq, d, dense_f, alg_f)
        bwd_ms = out["prefill_backward"]["ms_median"]
    if not args.no_kcache:
        out["decode_kcache"] = bench_kcache(W, dqr[:, 0], kcs, vcs, cl, qp, cut, G, ws, od, dec_alg, dmed)
    if not args.no_exact:
        out["exact_rule"] = bench_exact(W, qr, kr, v, dqr[:, 0], kcs, vcs, cl, qp, ws, od, theta, n, Hq, Hkv, d,
                                        Bd, L, q_pos, med["prefill"], dmed, bwd_ms)
    with_oracle = not args.no_cpu_baseline
    cpu_cfg = {}
    if with_oracle:
        log("bench: cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(qr, kr, v, n, Hq, d, G, theta, args.cpu_seconds)
        # the oracle on the rows the tests check, per workload: sampled rows of
        # the 32K prefill (with the labelled extrapolation), every sequence of
        # the decode
        import numpy as np
        import oracle as O
        from rope_positional_encoding_amd import synth
        threads = _oracle_threads()
        rows = synth.sample_rows(n, 256, 7, [c + e for c in cut for e in (0, 1)])
        done, dt, fl = oracle_prefill_rate(qr, kr, v, rows, O.dim_cutoffs_grouped(np.array(cut), G), threads)
        cpu_cfg["prefill32k_g16"] = {
            "rows": "%d sampled rows" % len(done), "seconds": round(dt, 2), "threads": threads,
            "dense_equiv_tflops": fl / dt / 1e12,
            "extrapolated_full_prefill_s": round(dt * (n * (n + 1) / 2.0) / float(np.sum(done + 1)), 1),
            "extrapolation": "x sum(i+1) over all rows / over the sampled rows"}
        ddt, kvb = oracle_decode_rate(dqr[:, 0], kc, vc, L, q_pos, cut, G, threads)
        cpu_cfg["decode32k"] = {"rows": "all %d sequences x %d keys" % (Bd, L), "seconds": round(ddt, 2),
                                "threads": threads, "kv_gbs_dense_equiv": kvb / ddt / 1e9}
    if not args.no_configs:
        out["configs"] = {}
        for name in PREFILL_CONFIGS:
            res, c = bench_prefill_config(W, name, gen, with_oracle,
                                          extra_flags=PREFILL_VARIANTS.get(name, ()))
            out["configs"][name] = res
            if c is not None:
                cpu_cfg[name] = c
    if with_oracle:
        out["cpu_baseline"]["per_config"] = cpu_cfg
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
