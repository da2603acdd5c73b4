"""Parity of the library's merging tree (ekh_merge_tree, host C++) with the oracle's.

Host code, so no GPU: the C ABI is called through the binding.  The bar is
exact: the same merges in the same order with bit-identical gains, on the
oracle's hand-worked cases and on random count matrices (sparse and dense, 2 to
200 clusters, several gamma, with exact ties).  Bad input is rejected.
"""
import numpy as np
import pytest

from exact_knn_hdbscan_amd import binding
from oracle import merge_tree as omt


def same(counts, gamma=1.0):
    got = binding.merge_tree(np.asarray(counts), gamma)
    want = omt.merge_tree(np.asarray(counts, np.int64), gamma)
    assert [(a, b) for a, b, _ in got] == [(a, b) for a, b, _ in want]
    np.testing.assert_array_equal(np.array([g for *_, g in got]), np.array([g for *_, g in want]))
    return got


def test_hand_worked():
    assert same([[5, 3, 0], [2, 5, 0], [0, 0, 5]]) == [(0, 1, -1 / 32), (0, 2, -3 / 8)]
    c = np.zeros((4, 4), np.int64)
    c[0, 1], c[1, 2], c[2, 3] = 1, 2, 3
    assert same(c, 0.0) == [(2, 3, 3 / 6), (1, 2, 2 / 6), (0, 1, 1 / 6)]
    c = np.zeros((3, 3), np.int64)
    c[0, 1], c[0, 2] = 1, 1
    assert same(c) == [(0, 1, 0.25), (0, 2, 0.125)]
    assert same(np.zeros((3, 3), np.int64)) == [(0, 1, 0.0), (0, 2, 0.0)]
    assert same(np.array([[7]])) == []


@pytest.mark.parametrize("C,density,gamma,seed", [(2, 1.0, 1.0, 0), (17, 0.3, 1.0, 1), (40, 0.1, 0.5, 2),
                                                  (40, 1.0, 1.0, 3), (200, 0.05, 1.0, 4), (64, 0.5, 0.0, 5)])
def test_random_counts(C, density, gamma, seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 6, (C, C)) * (rng.random((C, C)) < density)
    same(c, gamma)


def test_exact_ties():
    # a symmetric ring of equal weights: every first choice ties
    C = 12
    c = np.zeros((C, C), np.int64)
    for a in range(C):
        c[a, (a + 1) % C] = 3
    same(c)


def test_bad_input():
    with pytest.raises(binding.EkhError):
        binding.merge_tree(np.zeros((2, 2)), gamma=-1.0)
    with pytest.raises(binding.EkhError):
        binding.merge_tree(np.zeros((2, 2)), gamma=float("nan"))
