"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The pages print no worked example (no distances, lists or trees), so every pin
is a closed form, an invariant, a special case that reduces to a library
routine (scipy), or brute force on tiny inputs.  Each is chosen so that a
plausible slip in the oracle (a dropped term, a reversed tie rule, an
off-by-one in the core rank, a wrong edge order) fails at least one of them.
"""
import numpy as np
import pytest
from scipy.cluster.hierarchy import linkage
from scipy.sparse.csgraph import minimum_spanning_tree
from scipy.spatial import cKDTree
from scipy.spatial.distance import cdist, squareform

import oracle as _oracle
from exact_knn_hdbscan_amd import datagen
from treecheck import PathMax, is_spanning_tree, key_less, sort_edges

# ---------------------------------------------------------------- distances / kNN


def check_knn_distances_match_kdtree(orc):
    X = datagen.random_uniform(300, 7, seed=1)
    Y = datagen.random_uniform(200, 7, seed=2)
    idx, d2 = orc.knn(X, Y, 9)
    dd, ii = cKDTree(Y.T.astype(np.float64)).query(X.T.astype(np.float64), k=9)
    np.testing.assert_allclose(np.sqrt(d2), dd, rtol=1e-12, atol=1e-12)
    # random continuous data has no ties: the index lists agree too
    np.testing.assert_array_equal(idx, ii)


def check_knn_integer_grid_exact_and_ties_to_lower_index(orc):
    X = datagen.integer_grid(150, 5, seed=3, half_range=2)
    idx, d2 = orc.knn(X, X, 20)
    full = cdist(X.T.astype(np.float64), X.T.astype(np.float64), "sqeuclidean")
    for i in range(X.shape[1]):
        order = np.lexsort((np.arange(full.shape[1]), full[i]))  # (D^2, index)
        np.testing.assert_array_equal(idx[i], order[:20])
        np.testing.assert_array_equal(d2[i], full[i, order[:20]])
    assert np.any(d2[:, 1:] == d2[:, :-1]), "grid must contain ties for this pin"


def check_knn_collinear_closed_form(orc):
    n, s = 40, 0.5
    X = datagen.collinear(n, 3, spacing=s)
    k = 5
    idx, d2 = orc.knn(X, X, k)
    for i in range(n):
        # neighbours at |i - j| * s; on equal distance the lower index first
        exp = sorted(range(n), key=lambda j: (abs(i - j), j))[:k]
        np.testing.assert_array_equal(idx[i], exp)
        np.testing.assert_allclose(d2[i], [(abs(i - j) * s) ** 2 for j in exp], rtol=0, atol=0)


def check_knn_full_row_is_sorted_permutation(orc):
    X = datagen.integer_grid(60, 3, seed=4, half_range=1)
    idx, d2 = orc.knn(X, X, 60)
    for i in range(60):
        assert sorted(idx[i].tolist()) == list(range(60))
        assert np.all(np.diff(d2[i]) >= 0)
        eq = np.diff(d2[i]) == 0
        assert np.all(np.diff(idx[i])[eq] > 0), "equal distances must be in ascending index order"


def check_knn_k1_self_and_duplicates(orc):
    X = datagen.random_uniform(100, 4, seed=5)
    idx, d2 = orc.knn(X, X, 1)
    np.testing.assert_array_equal(idx[:, 0], np.arange(100))
    assert np.all(d2 == 0)
    D = datagen.duplicates(6, 4, seed=6, n_other=20)
    idx, d2 = orc.knn(D, D, 8)
    for i in range(6):
        np.testing.assert_array_equal(idx[i, :6], np.arange(6))
        assert np.all(d2[i, :6] == 0) and d2[i, 6] > 0


def check_knn_subset_orientation(orc):
    # queries are rows (all points); indices refer to the database Y
    X = datagen.random_uniform(80, 6, seed=7)
    Y = datagen.every_kth(X, 10)
    idx, d2 = orc.knn(X, Y, 3)
    assert idx.shape == (80, 3) and idx.max() < Y.shape[1]
    np.testing.assert_array_equal(idx[::10, 0], np.arange(8))  # subset members find themselves
    assert np.all(d2[::10, 0] == 0)


# ---------------------------------------------------------------- core distances


def check_core_collinear_closed_form(orc):
    n, s = 30, 2.0
    X = datagen.collinear(n, 2, spacing=s)
    core = orc.core_distances(X, 3)
    # self, left and right neighbour: interior core = s, ends reach two steps: 2s
    exp = np.full(n, s)
    exp[0] = exp[-1] = 2 * s
    np.testing.assert_array_equal(core, exp)
    np.testing.assert_array_equal(orc.core_distances(X, 1), np.zeros(n))
    core2 = orc.core_distances(X, 2)
    np.testing.assert_array_equal(core2, np.full(n, s))


def check_core_duplicates_zero(orc):
    D = datagen.duplicates(7, 5, seed=8, n_other=10)
    core = orc.core_distances(D, 7)
    assert np.all(core[:7] == 0) and np.all(core[7:] > 0)


def check_core_matches_kdtree_kth(orc):
    X = datagen.random_uniform(400, 6, seed=9)
    for ms in (1, 2, 5, 10):
        core = orc.core_distances(X, ms)
        dd, _ = cKDTree(X.T.astype(np.float64)).query(X.T.astype(np.float64), k=ms)
        kth = dd if ms == 1 else dd[:, ms - 1]
        np.testing.assert_allclose(core, kth, rtol=1e-12, atol=0)


# ---------------------------------------------------------------- minimum spanning tree


def _mst_both(orc, X, ms):
    core = orc.core_distances(X, ms)
    p = orc.mst_prim(X, core)
    k = orc.mst_kruskal(X, core)
    return core, p, k


def check_prim_equals_kruskal_exactly(orc, kind):
    if kind == "random":
        X, ms = datagen.random_uniform(300, 5, seed=10), 5
    elif kind == "grid":
        X, ms = datagen.integer_grid(250, 3, seed=11, half_range=2), 4
    elif kind == "dups":
        X, ms = datagen.duplicates(12, 4, seed=12, n_other=100), 3
    else:
        X, ms = datagen.spike_clips(300, 4, seed=13), 10
    core, (plo, phi, pw), (klo, khi, kw) = _mst_both(orc, X, ms)
    n = X.shape[1]
    assert is_spanning_tree(n, plo, phi) and is_spanning_tree(n, klo, khi)
    np.testing.assert_array_equal(plo, klo)
    np.testing.assert_array_equal(phi, khi)
    np.testing.assert_array_equal(pw, kw)
    assert np.all(plo < phi)


def check_mst_cycle_property_full_order(orc):
    """Every non-tree edge is larger, under (W, lo, hi), than every edge on the
    tree path between its endpoints: the certificate of the unique minimum tree."""
    X = datagen.integer_grid(200, 3, seed=14, half_range=2)
    core = orc.core_distances(X, 4)
    lo, hi, w = orc.mst_prim(X, core)
    M = orc.mutual_reachability_matrix(X, core)
    n = X.shape[1]
    a, b = np.triu_indices(n, 1)
    pm = PathMax(n, lo, hi)
    pos = pm.query(a, b)
    tw, tlo, thi = w[pos], lo[pos], hi[pos]
    is_tree = (tlo == a) & (thi == b)
    ew = M[a, b]
    bigger = key_less(tw, tlo, thi, ew, a, b)
    assert np.all(bigger | is_tree)
    assert is_tree.sum() == n - 1
    assert np.any((ew == tw) & ~is_tree), "the grid must contain weight ties for this pin"


def check_mst_collinear_ms2_path(orc):
    n, s = 25, 1.5
    X = datagen.collinear(n, 2, spacing=s)
    core, (lo, hi, w), _ = _mst_both(orc, X, 2)
    np.testing.assert_array_equal(lo, np.arange(n - 1))
    np.testing.assert_array_equal(hi, np.arange(1, n))
    assert w.sum() == pytest.approx((n - 1) * s, rel=1e-15)


def check_mst_collinear_ms3_tie_closed_form(orc):
    # cores: ends 2s, interior s.  0 joins through (0,1) (beats (0,2) on hi); the
    # last point n-1 joins through (n-3, n-1), which beats (n-2, n-1) on lo.
    n, s = 20, 1.0
    X = datagen.collinear(n, 2, spacing=s)
    core, (lo, hi, w), _ = _mst_both(orc, X, 3)
    exp = {(0, 1), (n - 3, n - 1)} | {(i, i + 1) for i in range(1, n - 2)}
    assert set(zip(lo.tolist(), hi.tolist())) == exp
    assert w.sum() == pytest.approx((n + 1) * s, rel=1e-15)


def check_mst_all_duplicates_star(orc):
    X = datagen.duplicates(30, 3, seed=15)
    core, (lo, hi, w), _ = _mst_both(orc, X, 4)
    np.testing.assert_array_equal(lo, np.zeros(29))
    np.testing.assert_array_equal(hi, np.arange(1, 30))
    assert np.all(w == 0)


def check_mst_ms1_is_euclidean_mst(orc):
    X = datagen.random_uniform(350, 4, seed=16)
    core = orc.core_distances(X, 1)
    assert np.all(core == 0)
    lo, hi, w = orc.mst_prim(X, core)
    E = cdist(X.T.astype(np.float64), X.T.astype(np.float64))
    total = minimum_spanning_tree(E).sum()
    assert w.sum() == pytest.approx(total, rel=1e-12)


def check_mst_weights_equal_single_linkage_heights(orc):
    X = datagen.spike_clips(200, 3, seed=17)
    core = orc.core_distances(X, 5)
    lo, hi, w = orc.mst_prim(X, core)
    M = orc.mutual_reachability_matrix(X, core)
    Z = linkage(squareform(M, checks=False), method="single")
    np.testing.assert_allclose(np.sort(w), np.sort(Z[:, 2]), rtol=1e-12)


def check_mst_degenerate_sizes(orc):
    X1 = datagen.random_uniform(1, 3, seed=18)
    lo, hi, w = orc.mst_prim(X1, np.zeros(1))
    assert lo.shape == (0,)
    X2 = datagen.random_uniform(2, 3, seed=19)
    core = orc.core_distances(X2, 2)
    lo, hi, w = orc.mst_prim(X2, core)
    assert (lo.tolist(), hi.tolist()) == ([0], [1])
    assert w[0] == pytest.approx(np.sqrt(orc.sqdist(X2, 0, X2, 1)))


def check_sort_helper_order(orc):
    lo, hi, w = sort_edges([3, 0, 1, 0], [4, 2, 2, 1], [1.0, 1.0, 0.5, 1.0])
    assert list(zip(w, lo, hi)) == [(0.5, 1, 2), (1.0, 0, 1), (1.0, 0, 2), (1.0, 3, 4)]


# ---------------------------------------------------------------- test entry points

CHECKS = [(name[len("check_"):], fn) for name, fn in list(globals().items())
          if name.startswith("check_") and name != "check_prim_equals_kruskal_exactly"]
KINDS = ["random", "grid", "dups", "clips"]


@pytest.mark.parametrize("name,fn", CHECKS, ids=[c[0] for c in CHECKS])
def test_pin(name, fn):
    fn(_oracle)


@pytest.mark.parametrize("kind", KINDS)
def test_prim_equals_kruskal_exactly(kind):
    check_prim_equals_kruskal_exactly(_oracle, kind)
