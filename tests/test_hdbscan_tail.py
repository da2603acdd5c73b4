"""Parity of the library's HDBSCAN tail (ekh_hdbscan_tail, host C++) with the oracle's.

The tail runs on the host (the HDBSCAN page puts it there), so these tests need
no GPU: they call the C ABI through the binding and compare with
oracle/hdbscan_tail.py entry for entry.  The bar is exact: the same condensed
tree (parents, children, sizes, lambda bit for bit), the same stabilities bit
for bit, the same selection and the same labels, on the oracle's own closed
forms, on oracle trees of clustered data (whose mutual-reachability weights
carry the built-in ties of the page's "ties" section), on a large random tree
with heavy ties, and on shuffled input.  Bad input must be rejected.
"""
import numpy as np
import pytest

import oracle
from exact_knn_hdbscan_amd import binding
from exact_knn_hdbscan_amd import datagen
from oracle import hdbscan_tail as otail

import test_hdbscan_tail_oracle as pins


def run_both(lo, hi, w, mcs):
    """lo, hi int, w float32 values; returns (library result, oracle result)."""
    lo = np.asarray(lo, np.int32)
    hi = np.asarray(hi, np.int32)
    w = np.asarray(w, np.float32)
    n = len(lo) + 1
    labels, tree = binding.hdbscan_tail(lo, hi, w, mcs, return_tree=True)
    ref = otail.hdbscan_tail(lo.astype(np.int64), hi.astype(np.int64), w.astype(np.float64), n, mcs)
    return labels, tree, ref


def assert_same(labels, tree, ref, n):
    ent = ref["entries"]
    assert tree["parent"].tolist() == [e[0] for e in ent]
    assert tree["child"].tolist() == [e[1] for e in ent]
    assert tree["size"].tolist() == [e[3] for e in ent]
    np.testing.assert_array_equal(tree["lambda"], np.array([e[2] for e in ent], np.float64))
    ids = sorted(ref["birth"])
    assert ids == list(range(n, n + tree["n_clusters"]))
    np.testing.assert_array_equal(tree["stability"], np.array([ref["stability"][c] for c in ids]))
    assert tree["n_selected"] == len(ref["selected"])
    np.testing.assert_array_equal(labels, ref["labels"].astype(np.int32))


@pytest.mark.parametrize("name", ["tie", "tie4", "line", "nested2", "nested125", "zero1", "zero2", "order"])
def test_closed_form_trees(name):
    trees = {
        "tie": (pins.TIE_TREE, 3), "tie4": (pins.TIE_TREE, 4),
        "line": ([(i, i + 1, 1.0) for i in range(4)] + [(4, 5, 10.0)] + [(i, i + 1, 2.0) for i in range(5, 9)], 3),
        "nested2": ([(i, i + 1, 1.0) for i in range(3)] + [(3, 4, 2.0)] + [(i, i + 1, 1.0) for i in range(4, 7)]
                    + [(7, 8, 22.0)] + [(i, i + 1, 1.0) for i in range(8, 11)], 4),
        "nested125": ([(i, i + 1, 1.0) for i in range(3)] + [(3, 4, 1.25)] + [(i, i + 1, 1.0) for i in range(4, 7)]
                      + [(7, 8, 22.0)] + [(i, i + 1, 1.0) for i in range(8, 11)], 4),
        "zero1": ([(0, 1, 0.0), (1, 2, 0.0), (3, 4, 0.0), (4, 5, 0.0), (2, 3, 1.0)], 3),
        "zero2": ([(0, 1, 0.0), (1, 5, 0.0), (2, 3, 0.0), (3, 4, 0.0), (4, 5, 0.0), (5, 6, 1.0)], 3),
        "order": ([(0, 1, 0.5), (1, 2, 0.5), (2, 3, 0.5), (4, 5, 0.5), (5, 6, 0.5), (6, 7, 0.5),
                   (1, 8, 1.0), (3, 4, 1.0)], 3),
    }
    lst, mcs = trees[name]
    lo, hi, w = pins._edges(lst)
    labels, tree, ref = run_both(lo, hi, w, mcs)
    assert_same(labels, tree, ref, len(lo) + 1)


@pytest.mark.parametrize("seed,ms,mcs", [(0, 10, 20), (1, 5, 15), (2, 3, 8), (3, 1, 5), (4, 10, 2)])
def test_oracle_trees_of_blobs(seed, ms, mcs):
    X = pins._blobs(seed, 120, 6, 5, noise=60)
    n = X.shape[1]
    lo, hi, w = pins._tree(X, ms)
    labels, tree, ref = run_both(lo, hi, w.astype(np.float32), mcs)
    assert_same(labels, tree, ref, n)
    assert tree["n_selected"] >= 2 or mcs > 100


@pytest.mark.parametrize("mcs", [5, 20, 60])
def test_oracle_tree_of_clips(mcs):
    wl = datagen.make("tiny_2000x60")
    X, ms = wl["X"], wl["min_samples"]
    core = oracle.core_distances(X, ms)
    lo, hi, w = oracle.mst_prim(X, core)
    labels, tree, ref = run_both(lo, hi, w.astype(np.float32), mcs)
    assert_same(labels, tree, ref, X.shape[1])


def _random_tree(n, seed, levels):
    rng = np.random.default_rng(seed)
    parent = np.array([rng.integers(0, i) for i in range(1, n)])
    child = np.arange(1, n)
    w = rng.integers(0, levels, n - 1).astype(np.float32) * 0.25  # many exact ties, zeros included
    lo, hi = np.minimum(parent, child), np.maximum(parent, child)
    return lo, hi, w


@pytest.mark.parametrize("n,levels,mcs", [(3000, 4, 10), (100000, 40, 50)])
def test_random_trees_with_heavy_ties(n, levels, mcs):
    lo, hi, w = _random_tree(n, 7, levels)
    labels, tree, ref = run_both(lo, hi, w, mcs)
    assert_same(labels, tree, ref, n)


def test_edge_order_of_input_is_irrelevant():
    X = pins._blobs(5, 100, 5, 4, noise=50)
    lo, hi, w = pins._tree(X, 5)
    w = w.astype(np.float32)
    base = binding.hdbscan_tail(lo, hi, w, 10, return_tree=True)
    perm = np.random.default_rng(1).permutation(len(lo))
    shuf = binding.hdbscan_tail(lo[perm], hi[perm], w[perm], 10, return_tree=True)
    np.testing.assert_array_equal(base[0], shuf[0])
    for k in ("parent", "child", "lambda", "size", "stability"):
        np.testing.assert_array_equal(base[1][k], shuf[1][k])


def test_single_point_and_bad_input():
    lab = binding.hdbscan_tail(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32), 5)
    assert lab.tolist() == [-1]
    lo, hi, w = np.array([0, 1], np.int32), np.array([1, 2], np.int32), np.array([1.0, 2.0], np.float32)
    assert binding.hdbscan_tail(lo, hi, w, 2).tolist() == [-1, -1, -1]
    bad = [
        (lo, hi, w, 1),                                                   # min_cluster_size < 2
        (np.array([0, 1], np.int32), np.array([1, 0], np.int32), w, 2),   # lo >= hi
        (np.array([0, 1], np.int32), np.array([1, 3], np.int32), w, 2),   # out of range
        (np.array([0, 0], np.int32), np.array([1, 1], np.int32), w, 2),   # cycle
        (lo, hi, np.array([1.0, -1.0], np.float32), 2),                   # negative weight
        (lo, hi, np.array([1.0, np.nan], np.float32), 2),                 # NaN
        (lo, hi, np.array([np.inf, 1.0], np.float32), 2),                 # infinite
    ]
    for a, b, c, m in bad:
        with pytest.raises(binding.EkhError) as ei:
            binding.hdbscan_tail(a, b, c, m)
        assert ei.value.code == binding.EKH_EINVAL
