"""The work models behind the bench's roofline figures, pinned by brute force
on small shapes (CPU): bench.prefill_flops (dense, algorithmic and executed
FLOPs of the prefill), bench.backward_flops (the backward's) and
bench.decode_bytes (dense, algorithmic and issued bytes of the decode).  Each
is recomputed here by enumerating every causal (query, key) pair, or every
cached key, with the oracle's per-dim cutoffs ([notes] section 2.1, Eq. (6),
grouped by section 2.3, Eq. (8)) and, for the tile-granular counts, with the
oracle's tile classifier."""
import numpy as np
import pytest

import bench
import oracle as O
import rope_positional_encoding_amd as W

SHAPES = [(300, 4, 128, 16, 300.0), (257, 2, 64, 32, 100.0), (190, 3, 128, 32, 1e4), (129, 1, 64, 16, 30.0)]


def _pairs(n):
    i, j = np.tril_indices(n)
    return i - j                         # the distance of every causal pair


@pytest.mark.parametrize("n,Hq,d,G,theta", SHAPES)
def test_prefill_flops_by_pair_enumeration(n, Hq, d, G, theta):
    cut = O.group_cutoffs(theta, d, G)
    dim_cut = O.dim_cutoffs_grouped(cut, G)
    dist = _pairs(n)
    kept_dims = (dist[:, None] <= dim_cut[None, :]).sum(axis=1)      # per pair
    dense = Hq * len(dist) * 4.0 * d                                  # QK + PV over all dims
    alg = Hq * float((2.0 * kept_dims + 2.0 * d).sum())              # kept QK dims + all PV dims
    bd, ba, be = bench.prefill_flops(n, Hq, 1, d, G, [int(c) for c in cut])
    assert bd == pytest.approx(dense, rel=1e-12)
    assert ba == pytest.approx(alg, rel=1e-12)
    # executed: every visited (BM x BN) tile does its PV and the QK of its
    # non-skipped groups in full, whatever its causal mask
    BM, BN = W.prefill_tiling(d, G)
    c, vis = O.prefill_tile_counts(n, BM, BN, cut)
    exe = Hq * (vis * 2.0 * BM * BN * d + (c[:, 1] + c[:, 2]).sum() * 2.0 * BM * BN * G)
    assert be == pytest.approx(exe, rel=1e-12)
    assert alg <= be


@pytest.mark.parametrize("n,Hq,d,G,theta", SHAPES)
def test_backward_flops_by_pair_enumeration(n, Hq, d, G, theta):
    cut = O.group_cutoffs(theta, d, G)
    dim_cut = O.dim_cutoffs_grouped(cut, G)
    dist = _pairs(n)
    kept_dims = (dist[:, None] <= dim_cut[None, :]).sum(axis=1)
    # S, dK, dQ over the kept dims; dP and dV over all dims
    alg = Hq * float((3 * 2.0 * kept_dims + 2 * 2.0 * d).sum())
    dense = Hq * len(dist) * 5 * 2.0 * d
    fd, fa, _ = bench.prefill_flops(n, Hq, 1, d, G, [int(c) for c in cut])
    bd, ba = bench.backward_flops(fd, fa)
    assert bd == pytest.approx(dense, rel=1e-12)
    assert ba == pytest.approx(alg, rel=1e-12)


@pytest.mark.parametrize("L,q_pos,Hkv,Hq,d,G,theta", [(1000, 999, 2, 8, 128, 16, 300.0), (700, 700, 1, 4, 64, 32, 100.0),
                                                      (513, 514, 4, 4, 128, 32, 1e4), (1, 0, 1, 1, 64, 16, 30.0)])
def test_decode_bytes_by_key_enumeration(L, q_pos, Hkv, Hq, d, G, theta):
    cut = O.group_cutoffs(theta, d, G)
    dim_cut = O.dim_cutoffs_grouped(cut, G)
    dist = q_pos - np.arange(L)
    kept_k = (dist[:, None] <= dim_cut[None, :]).sum()               # kept K elements of one kv head
    qo = 2 * 2.0 * Hq * d                                            # q read, o written (bf16)
    dense = Hkv * 2 * 2.0 * L * d
    alg = Hkv * (2.0 * kept_k + 2.0 * L * d) + qo
    bd, ba, bi = bench.decode_bytes(L, q_pos, Hkv, Hq, 1, d, G, [int(c) for c in cut])
    assert bd == pytest.approx(dense, rel=1e-12)
    assert ba == pytest.approx(alg, rel=1e-12)
    # issued: every non-skipped group of every visited BN-key block, all V
    BN = W.decode_tiling(d, G)
    c, vis = O.decode_tile_counts(q_pos, L, BN, cut)
    issued = Hkv * ((c[:, 1] + c[:, 2]).sum() * BN * 2.0 * G + 2.0 * L * d) + qo
    assert bi == pytest.approx(issued, rel=1e-12)
    assert ba <= bi + 1e-9
