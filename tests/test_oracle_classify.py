"""Pins for tile classification ([notes] §2.3 table; thread 6/7).

The oracle's l_D/r_D formula is checked against the pages' wording applied by
brute force to every causal pair of a tile, on random tiles and on whole tile
grids (ragged tails included)."""
import numpy as np
import pytest

import oracle as O


def test_formula_matches_pair_enumeration_random_tiles():
    rng = np.random.default_rng(31)
    for _ in range(400):
        BM, BN = int(rng.integers(1, 20)), int(rng.integers(1, 20))
        i0, j0 = int(rng.integers(0, 120)), int(rng.integers(0, 120))
        qpos = np.arange(i0, i0 + BM)
        kpos = np.arange(j0, j0 + BN)
        cut = np.sort(rng.integers(0, 140, size=int(rng.integers(1, 9))))
        bf = O.classify_bruteforce(qpos, kpos, cut)
        if bf is None:
            assert j0 > i0 + BM - 1
            continue
        l_D = max(0, i0 - (j0 + BN - 1))
        r_D = (i0 + BM - 1) - j0
        assert np.array_equal(O.classify(l_D, r_D, cut), bf)


def test_classes_form_skip_prefix_partial_middle_full_suffix():
    rng = np.random.default_rng(32)
    for _ in range(200):
        cut = np.sort(rng.integers(0, 1000, size=8))
        l_D = int(rng.integers(0, 1000))
        r_D = l_D + int(rng.integers(0, 200))
        c = O.classify(l_D, r_D, cut)
        assert np.all(np.diff(c) >= 0)
        splitL = int((cut < l_D).sum())
        splitR = int((cut < r_D).sum())
        assert np.all(c[:splitL] == O.SKIP)
        assert np.all(c[splitL:splitR] == O.PARTIAL)
        assert np.all(c[splitR:] == O.FULL)


def _grid_bruteforce(n, BM, BN, cut):
    counts = np.zeros((len(cut), 3), dtype=np.int64)
    visited = 0
    for i0 in range(0, n, BM):
        for j0 in range(0, n, BN):
            bf = O.classify_bruteforce(np.arange(i0, min(n, i0 + BM)),
                                       np.arange(j0, min(n, j0 + BN)), cut)
            if bf is None:
                continue
            visited += 1
            for g, c in enumerate(bf):
                counts[g, c] += 1
    return counts, visited


@pytest.mark.parametrize("n,BM,BN", [(256, 32, 32), (200, 32, 32), (97, 16, 8), (130, 64, 32)])
def test_prefill_grid_counts_match_bruteforce(n, BM, BN):
    for cut in (np.array([6, 19, 62, 198]), np.array([47, 471, 4711, 47117]),
                np.array([0, 0, 31, 33, 64, 65, 500, 10 ** 9])):
        c1, v1 = O.prefill_tile_counts(n, BM, BN, cut)
        c2, v2 = _grid_bruteforce(n, BM, BN, cut)
        assert v1 == v2
        assert np.array_equal(c1, c2)
        assert np.all(c1.sum(1) == v1)


@pytest.mark.parametrize("q_pos,L,BN", [(300, 300, 32), (299, 300, 32), (1000, 777, 16)])
def test_decode_grid_counts_match_bruteforce(q_pos, L, BN):
    cut = np.array([6, 19, 62, 198, 400, 10 ** 9])
    c1, v1 = O.decode_tile_counts(q_pos, L, BN, cut)
    counts = np.zeros_like(c1)
    nb = 0
    for j0 in range(0, L, BN):
        bf = O.classify_bruteforce([q_pos], np.arange(j0, min(L, j0 + BN)), cut)
        nb += 1
        for g, c in enumerate(bf):
            counts[g, c] += 1
    assert v1 == nb
    assert np.array_equal(c1, counts)
