"""CPU tests of the C ABI: the library loads and exports every function the
header declares; host-only calls (cutoff table, tiling, host tile classifier)
agree bit-exactly with the oracle; invalid arguments are rejected before any
HIP call (so these run without a GPU)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle as O
import rope_positional_encoding_amd as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "waveprune.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wp_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 13
    L = ctypes.CDLL(W.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(names) == set(W._SIGNATURES), "binding signatures out of sync with the header"


@pytest.mark.parametrize("theta", [10.0, 100.0, 500.0, 1e4, 5e5, 1e6, 1e7])
@pytest.mark.parametrize("d_h", [8, 16, 64, 128])
@pytest.mark.parametrize("s", [1.0, 2.0, 4.0, 8.0])
def test_group_cutoffs_match_oracle(theta, d_h, s):
    for G in (2, 4, 8, 16, 32):
        if d_h % G:
            continue
        got = W.group_cutoffs(theta, d_h, G, s)
        ref = O.group_cutoffs(theta, d_h, G, s)
        assert got == [int(v) for v in ref]


def test_group_cutoffs_clamp_never_prune():
    # d_h = 128, theta = 1e12, scale 1e6: low channels exceed 2^31 - 1
    got = W.group_cutoffs(1e12, 128, 16, 1e6)
    assert got[-1] == W.NEVER_PRUNE
    assert got == [int(v) for v in O.group_cutoffs(1e12, 128, 16, 1e6)]


def _i32(vals):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def _i64(vals):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _ramp_scaled_freqs(theta, d_h, s, lo=0.25, hi=0.75):
    """A per-channel scaled schedule: the first `lo` fraction of channels
    keep their frequency, the last (1 - hi) are divided by s, and the ones in
    between are divided by a factor that ramps linearly from 1 to s."""
    n = d_h // 2
    f = O.frequencies(theta, d_h)
    out = []
    for c in range(n):
        t = min(1.0, max(0.0, (c / (n - 1) - lo) / (hi - lo)))
        out.append(f[c] / (1.0 + t * (s - 1.0)))
    return out


@pytest.mark.parametrize("alpha", [0.5, 1.0, 1.7, 2.0, 2.5, 4.0, math.inf])
@pytest.mark.parametrize("trunc", [None, 0, 1, 8, 40])
def test_general_cutoffs_match_oracle(alpha, trunc):
    cases = [list(O.frequencies(1e6, 128)), list(O.frequencies(1e4, 64, 4.0)),
             _ramp_scaled_freqs(1e6, 128, 8.0), _ramp_scaled_freqs(5e5, 64, 32.0)]
    for f in cases:
        n_ch = len(f)
        k = n_ch if trunc is None else min(trunc, n_ch)
        ch = O.cutoffs_from_freqs(f, alpha, k)
        for G in (2, 4, 16, 32):
            if (2 * n_ch) % G:
                continue
            got = W.cutoffs_from_freqs(f, G, alpha, k)
            assert got == [int(v) for v in O.group_max(ch, G)], (alpha, k, G)


def test_general_cutoffs_equal_theta_table():
    for theta, d_h, s in [(1e4, 64, 1.0), (1e6, 128, 1.0), (1e6, 128, 4.0)]:
        f = list(O.frequencies(theta, d_h, s))
        for G in (16, 32):
            assert W.cutoffs_from_freqs(f, G) == W.group_cutoffs(theta, d_h, G, s)


def test_general_cutoffs_validation():
    f = list(O.frequencies(1e6, 128))
    L = W.lib()
    out = (ctypes.c_int32 * 8)()
    arr = (ctypes.c_double * 64)(*f)
    assert L.wp_cutoffs_from_freqs(None, 64, 2.0, 64, 16, out, 8) == -1
    assert L.wp_cutoffs_from_freqs(arr, 64, 2.0, 64, 16, None, 8) == -1
    assert L.wp_cutoffs_from_freqs(arr, 0, 2.0, 0, 16, out, 0) == -2
    assert L.wp_cutoffs_from_freqs(arr, 64, 2.0, 65, 16, out, 8) == -2      # trunc > n_ch
    assert L.wp_cutoffs_from_freqs(arr, 64, 2.0, -1, 16, out, 8) == -2
    assert L.wp_cutoffs_from_freqs(arr, 64, 2.0, 64, 12, out, 8) == -2      # G does not divide 128
    assert L.wp_cutoffs_from_freqs(arr, 64, 2.0, 64, 16, out, 7) == -2      # out_len
    assert L.wp_cutoffs_from_freqs(arr, 64, 0.0, 64, 16, out, 8) == -6      # alpha
    assert L.wp_cutoffs_from_freqs(arr, 64, math.nan, 64, 16, out, 8) == -6
    bad = (ctypes.c_double * 64)(*([0.0] + f[1:]))
    assert L.wp_cutoffs_from_freqs(bad, 64, 2.0, 64, 16, out, 8) == -6      # zero frequency
    # increasing frequencies give a decreasing table: rejected, out untouched
    rev = (ctypes.c_double * 64)(*reversed(f))
    for i in range(8):
        out[i] = -7
    assert L.wp_cutoffs_from_freqs(rev, 64, 2.0, 64, 16, out, 8) == -6
    assert list(out) == [-7] * 8
    assert b"non-decreasing" in L.wp_last_error()


def test_kcache_layout_definition_and_printed_table():
    # group g keeps min(Lmax, D'_g + 1) slots; the cutoffs are the printed
    # table at theta = 1e6, d_h = 128, G = 16 (28/160/900/5063/28472/...)
    cut = W.group_cutoffs(1e6, 128, 16)
    caps, offs = W.kcache_layout(32768, 128, 16, cut)
    assert caps == [29, 161, 901, 5064, 28473, 32768, 32768, 32768]
    assert offs == [0] + list(np.cumsum([c * 16 for c in caps]))
    for Lmax, d, G, cut in [(1, 64, 16, [0, 5, 9, 2**31 - 1]), (1000, 128, 32, [3, 999, 1000, 5000]),
                            (77, 64, 32, [76, 2**31 - 1])]:
        caps, offs = W.kcache_layout(Lmax, d, G, cut)
        assert caps == [min(Lmax, c + 1) for c in cut]
        assert offs[-1] == sum(c * G for c in caps)


def test_kcache_validation_codes():
    L = W.lib()
    cut = _i32(W.group_cutoffs(1e4, 128, 16))
    caps = (ctypes.c_int32 * 8)()
    offs = (ctypes.c_int64 * 9)()
    assert L.wp_kcache_layout(100, 128, 16, None, caps, offs) == -1
    assert L.wp_kcache_layout(0, 128, 16, cut, caps, offs) == -2
    assert L.wp_kcache_layout(100, 96, 16, cut, caps, offs) == -3
    bad = _i32([5, 4, 6, 7, 8, 9, 10, 11])
    assert L.wp_kcache_layout(100, 128, 16, bad, caps, offs) == -6
    assert L.wp_kcache_layout(100, 128, 16, cut, caps, offs) == 0
    total = offs[8]
    F = ctypes.c_void_p(1 << 20)      # never dereferenced: every call below fails validation
    ks = _i64([4096, 1024, 128])
    ss = _i64([total * 8, total])
    assert L.wp_kcache_append(None, 1, 4, 8, 128, ks, F, F, ss, 100, cut, 16, None) == -1
    assert L.wp_kcache_append(F, 1, 0, 8, 128, ks, F, F, ss, 100, cut, 16, None) == -2
    assert L.wp_kcache_append(F, 1, 101, 8, 128, ks, F, F, ss, 100, cut, 16, None) == -2   # T > Lmax
    assert L.wp_kcache_append(F, 1, 4, 8, 128, ks, F, F, _i64([total * 8, total - 16]), 100, cut, 16,
                              None) == -2                                                    # store stride
    assert L.wp_kcache_append(F, 1, 4, 8, 128, ks, F, F, _i64([total * 8, total + 4]), 100, cut, 16,
                              None) == -4                                                    # stride % 8
    assert L.wp_kcache_append(ctypes.c_void_p((1 << 20) + 8), 1, 4, 8, 128, ks, F, F, ss, 100, cut, 16,
                              None) == -4
    assert L.wp_kcache_append(F, 1, 4, 8, 128, ks, F, F, ss, (1 << 24) + 1, cut, 16, None) == -2
    st9 = _i64([4096, 128, total * 8, total, 1024 * 100, 1024, 128, 4096, 128])
    args = [F, F, F, F, F, F, 1, 100, 32, 8, 128, st9, cut, 16, 0, F, 1 << 30, 0, None, None]
    bad_args = list(args)
    bad_args[17] = 1      # WP_FLAG_DENSE is rejected for the compact store
    assert L.wp_decode_kcache(*bad_args) == -6
    bad_args = list(args)
    bad_args[12] = None   # cutoffs are required
    assert L.wp_decode_kcache(*bad_args) == -1
    bad_args = list(args)
    bad_args[11] = _i64([4096, 128, total * 8, total - 16, 1024 * 100, 1024, 128, 4096, 128])
    assert L.wp_decode_kcache(*bad_args) == -2


def test_tiling_queries():
    assert W.prefill_tiling(128, 16) == (32, 64)
    assert W.prefill_tiling(64, 32) == (32, 64)
    assert W.decode_tiling(128, 16) == 32
    with pytest.raises(W.WPError) as e:
        W.prefill_tiling(96, 16)
    assert e.value.status == -3


@pytest.mark.parametrize("n", [1, 31, 32, 33, 256, 1000, 4096])
@pytest.mark.parametrize("cfg", [(64, 16, 1e4, 1.0), (128, 16, 1e6, 1.0), (128, 32, 1e6, 1.0),
                                 (128, 16, 1e6, 4.0), (64, 32, 100.0, 1.0), (128, 16, 30.0, 1.0),
                                 (128, 2, 1e4, 1.0), (128, 4, 1e6, 1.0), (64, 8, 300.0, 1.0)])
def test_host_prefill_classifier_matches_oracle(n, cfg):
    d_h, G, theta, s = cfg
    cut = [int(v) for v in O.group_cutoffs(theta, d_h, G, s)]
    BM, BN = W.prefill_tiling(d_h, G)
    got = W.prefill_tile_counts(n, d_h, G, cut)
    c, v = O.prefill_tile_counts(n, BM, BN, np.array(cut))
    assert got == list(c.ravel()) + [v]


def test_host_prefill_classifier_32k_and_128k():
    for n, s in ((32768, 1.0), (131072, 4.0)):
        cut = [int(v) for v in O.group_cutoffs(1e6, 128, 16, s)]
        got = W.prefill_tile_counts(n, 128, 16, cut)
        BM, BN = W.prefill_tiling(128, 16)
        c, v = O.prefill_tile_counts(n, BM, BN, np.array(cut))
        assert got == list(c.ravel()) + [v]


@pytest.mark.parametrize("q_pos,L", [(32768, 32768), (32767, 32768), (5000, 33), (40, 1), (0, 1)])
def test_host_decode_classifier_matches_oracle(q_pos, L):
    for d_h, G, theta in ((128, 16, 1e6), (128, 32, 1e6), (64, 16, 1e3), (128, 2, 1e4), (64, 4, 1e3)):
        cut = [int(v) for v in O.group_cutoffs(theta, d_h, G)]
        got = W.decode_tile_counts(q_pos, L, d_h, G, cut)
        c, v = O.decode_tile_counts(q_pos, L, W.decode_tiling(d_h, G), np.array(cut))
        assert got == list(c.ravel()) + [v]


def test_classifier_rejects_bad_tables():
    with pytest.raises(W.WPError) as e:
        W.prefill_tile_counts(100, 128, 16, [5, 4, 6, 7, 8, 9, 10, 11])
    assert e.value.status == -6
    with pytest.raises(W.WPError) as e:
        W.prefill_tile_counts(100, 128, 16, [-1, 4, 6, 7, 8, 9, 10, 11])
    assert e.value.status == -6


# ---- validation happens before any HIP call: fake aligned device pointers ----
FAKE = ctypes.c_void_p(0x7F0000000000)   # never dereferenced: every call below fails validation


def _strides(n):
    # plausible element strides (multiples of 8, token strides >= d_h = 128)
    return (ctypes.c_int64 * n)(*([1024] * n))


def _prefill(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, n=64, Hq=4, Hkv=2, d_h=128,
                strides=_strides(12), cut=(ctypes.c_int32 * 8)(*range(8)), G=16, flags=0,
                counters=None, stream=None)
    args.update(kw)
    return W.lib().wp_prefill(*args.values())


def test_prefill_validation_codes():
    assert _prefill(q=None) == -1
    assert _prefill(d_h=96) == -3
    assert _prefill(G=12) == -3
    assert _prefill(Hq=3) == -2
    assert _prefill(n=0) == -2
    assert _prefill(q=ctypes.c_void_p(0x7F0000000008)) == -4
    st = _strides(12)
    st[4] = 12
    assert _prefill(strides=st) == -4
    assert _prefill(cut=(ctypes.c_int32 * 8)(9, 8, 7, 6, 5, 4, 3, 2)) == -6
    assert "non-decreasing" in W.lib().wp_last_error().decode()
    assert _prefill(cut=None) == -1
    assert _prefill(flags=2) == -1                       # COUNT without counters
    assert _prefill(flags=8) == -6                       # unknown flag
    st = _strides(12)
    st[4] = 64                                           # k token stride < d_h
    assert _prefill(strides=st) == -2
    st = _strides(12)
    st[7] = 1 << 25                                      # one 64-token V tile > 2 GiB
    assert _prefill(strides=st, n=200) == -2
    # 64 KB per token: a 4 GiB sequence at n = 65536 passes the span checks
    # (a tile spans 4 MB) and stops at the cutoff table, checked after them
    st = _strides(12)
    st[4] = st[7] = 1 << 15
    assert _prefill(strides=st, n=1 << 16, cut=(ctypes.c_int32 * 8)(9, 8, 7, 6, 5, 4, 3, 2)) == -6
    assert "non-decreasing" in W.lib().wp_last_error().decode()


def _decode(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, cl=FAKE, qp=FAKE, B=2, Lmax=100, Hq=4, Hkv=2,
                d_h=128, strides=_strides(10), cut=(ctypes.c_int32 * 8)(*range(8)), G=16,
                splits=0, ws=FAKE, ws_bytes=1 << 30, flags=0, counters=None, stream=None)
    args.update(kw)
    return W.lib().wp_decode(*args.values())


def test_decode_cache_span_limits():
    # every 32-key block is read through its own 32-bit buffer resources, so
    # the cache length is not limited by the byte span: 2^20 + 1 and 2^22 keys
    # at a 2 KB token stride (1 M tokens x 8 kv heads x 128 dims is 2 GiB of K
    # per sequence) pass validation (stopped here by the small workspace);
    # a token stride whose 32-token block spans 2^31 bytes is rejected
    st = _strides(10)
    st[3] = st[6] = 8 * 128                              # k_t, v_t in elements
    for L in (1 << 20, (1 << 20) + 1, 1 << 22):
        assert _decode(B=1, Lmax=L, Hq=8, Hkv=2, strides=st, ws_bytes=16) == -5
    st[3] = 1 << 26                                      # 128 MB per token: a block spans 4 GB
    assert _decode(B=1, Lmax=100, Hq=8, Hkv=2, strides=st, ws_bytes=16) == -2
    st = _strides(10)
    st[6] = (1 << 30) + 8                                # byte stride past 2^31
    assert _decode(B=1, Lmax=1, Hq=8, Hkv=2, strides=st, ws_bytes=16) == -2


def test_decode_validation_codes():
    assert _decode(ws=None) == -1
    assert _decode(d_h=80) == -3
    # more than 32 query heads per kv head are accepted (they run in passes of
    # 32): validation stops at the small workspace
    assert _decode(Hq=64, Hkv=2, ws_bytes=16) == -5
    assert _decode(ws_bytes=16) == -5
    assert _decode(ws=ctypes.c_void_p(0x7F0000000010)) == -4
    assert _decode(splits=-1) == -6
    assert _decode(Lmax=0) == -2


def test_rope_validation_codes():
    L = W.lib()
    s3 = _strides(3)
    assert L.wp_rope_apply(FAKE, 2, FAKE, 1, 8, 2, 128, s3, s3, None, 1e4, 1.0, None) == -6
    assert L.wp_rope_apply(FAKE, 0, FAKE, 1, 8, 2, 128, s3, s3, None, -1.0, 1.0, None) == -6
    assert L.wp_rope_apply(FAKE, 0, FAKE, 1, 8, 2, 128, s3, s3, None, 1e4, 0.0, None) == -6
    assert L.wp_rope_apply(FAKE, 0, FAKE, 1, 8, 2, 96, s3, s3, None, 1e4, 1.0, None) == -3
    assert L.wp_rope_apply(FAKE, 1, FAKE, 1, 8, 2, 128, s3, s3, None, 1e4, 1.0, None) == -6  # f32 in place
    assert L.wp_rope_apply(None, 0, FAKE, 1, 8, 2, 128, s3, s3, None, 1e4, 1.0, None) == -1


def test_status_strings():
    L = W.lib()
    for s in range(0, -8, -1):
        assert L.wp_status_string(s)
    assert L.wp_version().decode().count(".") == 2


def _backward(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dout=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, n=64,
                Hq=4, Hkv=2, d_h=128, strides=_strides(24), cut=(ctypes.c_int32 * 8)(*range(8)), G=16,
                flags=0, ws=FAKE, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return W.lib().wp_prefill_backward(*args.values())


def test_backward_workspace_size():
    # two floats per query row (its base-2 LSE and Dsum), rounded up to 256 bytes
    L = W.lib()
    assert L.wp_prefill_backward_workspace_size(2, 1000, 8) == 2 * 1000 * 8 * 8
    assert L.wp_prefill_backward_workspace_size(1, 3, 1) == 256
    assert L.wp_prefill_backward_workspace_size(0, 10, 1) == 0


def test_backward_validation_codes():
    # every call here fails validation, so no kernel is launched
    assert _backward(lse=None) == -1
    assert _backward(dv=None) == -1
    assert _backward(d_h=96) == -3
    assert _backward(Hq=3) == -2
    assert _backward(n=0) == -2
    assert _backward(ws_bytes=1024) == -5                # need 1 * 4 * 64 * 8 bytes
    assert _backward(flags=2) == -6                      # only WP_FLAG_DENSE is known
    assert _backward(cut=None) == -1
    assert _backward(cut=(ctypes.c_int32 * 8)(9, 8, 7, 6, 5, 4, 3, 2)) == -6
    assert _backward(ws=ctypes.c_void_p(0x7F0000000010)) == -4
    st = _strides(24)
    st[13] = 64                                          # dO token stride < d_h
    assert _backward(strides=st) == -2


def test_fine_groups_scope():
    # G = 2, 4, 8 (down to one cutoff per channel) run in prefill, decode and
    # the backward pass; the compact K store takes G = 16 or 32 only
    for G in (2, 4, 8):
        assert W.prefill_tiling(128, G) == (32, 64)
        assert W.decode_tiling(64, G) == 32
        # the group size is accepted: validation stops at the small workspace
        cutg = (ctypes.c_int32 * (128 // G))(*range(128 // G))
        assert _backward(G=G, cut=cutg, ws_bytes=1024) == -5
    assert _backward(G=12, cut=(ctypes.c_int32 * 64)(*range(64))) == -3
    L = W.lib()
    caps = (ctypes.c_int32 * 64)()
    offs = (ctypes.c_int64 * 65)()
    cut = (ctypes.c_int32 * 64)(*range(64))
    assert L.wp_kcache_layout(1000, 128, 2, cut, caps, offs) == -3
    assert L.wp_kcache_layout(1000, 128, 8, cut, caps, offs) == -3
    with pytest.raises(W.WPError) as e:
        W.prefill_tiling(128, 12)
    assert e.value.status == -3
