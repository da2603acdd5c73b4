"""GPU parity of ekh_mst_boruvka against the float64 oracle (Prim)."""
import numpy as np
import pytest

import exact_knn_hdbscan_amd as ekh
import oracle
from exact_knn_hdbscan_amd import datagen
from gpu_util import dev, host, say
from parity import check_mst, check_tree_shape

pytestmark = pytest.mark.gpu


def gpu_mst(X, ms, flags=0, with_lists=True, stats=False):
    Xg = dev(X)
    core, ni, nd2 = ekh.core_distances(Xg, ms, return_neighbours=True)
    if with_lists:
        out = ekh.mst_boruvka(Xg, core, ms, ni, nd2, flags=flags, return_stats=True)
    else:
        out = ekh.mst_boruvka(Xg, core, ms, flags=flags, return_stats=True)
    lo, hi, w, st = out
    res = (host(lo), host(hi), host(w))
    return (res + (st,)) if stats else res


def test_mst_tiny():
    X = datagen.make("tiny_2000x60")["X"]
    say("mst tiny 2000x60 ms=10")
    lo, hi, w, st = gpu_mst(X, 10, stats=True)
    say("stats", st)
    rep = {}
    check_mst(X, 10, lo, hi, w, report=rep)
    say("report", rep)


@pytest.mark.parametrize("n,d,ms", [(700, 5, 4), (1001, 61, 10), (513, 3, 1), (400, 2, 2), (600, 150, 3)])
def test_mst_integer_grid_identical(n, d, ms):
    """Integer coordinates keep every D2 exact and every weight comparison
    identical in float32 and float64, so the trees must be equal edge for edge."""
    X = datagen.integer_grid(n, d, seed=n + d, half_range=2)
    say("mst integer n=%d d=%d ms=%d" % (n, d, ms))
    lo, hi, w = gpu_mst(X, ms)
    core = oracle.core_distances(X, ms)
    olo, ohi, ow = oracle.mst_prim(X, core)
    np.testing.assert_array_equal(lo, olo)
    np.testing.assert_array_equal(hi, ohi)
    np.testing.assert_array_equal(w, ow.astype(np.float32))


def test_mst_integer_grid_large_with_ties():
    """20,000 integer points in 3-D (coordinates -6..6): heavy exact ties in
    every round, and a last round whose largest component is scanned against
    the points outside it only.  Edge for edge equal to the oracle's Prim, and
    to the tree with full scans (flag 4)."""
    X = datagen.integer_grid(20000, 3, seed=20003, half_range=6)
    lo, hi, w, st = gpu_mst(X, 4, stats=True)
    say("scanned %s, largest component apart %s" % (st["scanned"], st["scanned_giant"]))
    assert sum(st["scanned_giant"]) > 0
    core = oracle.core_distances(X, 4)
    olo, ohi, ow = oracle.mst_prim(X, core)
    np.testing.assert_array_equal(lo, olo)
    np.testing.assert_array_equal(hi, ohi)
    np.testing.assert_array_equal(w, ow.astype(np.float32))
    for a, b in zip((lo, hi, w), gpu_mst(X, 4, flags=4)):
        np.testing.assert_array_equal(a, b)


def test_mst_closed_forms():
    n = 150
    say("mst collinear ms=2 / ms=3, duplicates star")
    X = datagen.collinear(n, 61, spacing=1.0)
    lo, hi, w = gpu_mst(X, 2)
    np.testing.assert_array_equal(lo, np.arange(n - 1))
    np.testing.assert_array_equal(hi, np.arange(1, n))
    assert w.sum() == n - 1
    lo, hi, w = gpu_mst(X, 3)
    exp = {(0, 1), (n - 3, n - 1)} | {(i, i + 1) for i in range(1, n - 2)}
    assert set(zip(lo.tolist(), hi.tolist())) == exp
    D = datagen.duplicates(40, 61, seed=9)
    lo, hi, w = gpu_mst(D, 5)
    np.testing.assert_array_equal(lo, np.zeros(39))
    np.testing.assert_array_equal(hi, np.arange(1, 40))
    assert np.all(w == 0)


@pytest.mark.parametrize("ms", [1, 5, 10])
def test_mst_clips(ms):
    X = datagen.spike_clips(4000, 12, seed=ms, noise_frac=0.03)
    say("mst clips 4000x61 ms=%d" % ms)
    lo, hi, w, st = gpu_mst(X, ms, stats=True)
    say("stats", {k: st[k] for k in ("rounds", "n_components", "resolved", "skipped", "scanned")})
    rep = {}
    check_mst(X, ms, lo, hi, w, report=rep)
    say("report", rep)


def test_pruning_is_exact():
    """The tree with every exact shortcut equals the tree without any, bit for
    bit, on clip-like data with duplicates ("Exact shortcuts": the test
    pruning_is_exact builds it both ways); so does the tree whose largest
    component is scanned against all points (flag 4) instead of only the points
    outside it."""
    base = datagen.spike_clips(3000, 10, seed=3)
    X = np.ascontiguousarray(np.concatenate([base, base[:, :200], base[:, 1000:1100]], axis=1))
    say("pruning is exact, n=%d" % X.shape[1])
    ref = gpu_mst(X, 10, flags=7)
    giant = 0
    for flags in (0, 1, 2, 3, 4):
        got = gpu_mst(X, 10, flags=flags, stats=True)
        for a, b in zip(got[:3], ref):
            np.testing.assert_array_equal(a, b)
        giant += sum(got[3]["scanned_giant"]) if not flags & 4 else 0
        if flags & 4:
            assert sum(got[3]["scanned_giant"]) == 0
    say("points scanned against the largest component's complement: %d" % giant)
    assert giant > 0
    got = gpu_mst(X, 10, with_lists=False)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    check_mst(X, 10, *ref)


@pytest.mark.parametrize("d", [9, 33, 90, 100, 129, 170, 200, 240, 256])
def test_mst_dimensions(d):
    """The scan kernel across its instantiations (QM = 4 ceil(d / 16) k-steps;
    32-row tiles up to d = 224, 16-row tiles beyond)."""
    X = datagen.gaussian_mixture(1500, d, 6, seed=d)
    say("mst d=%d" % d)
    lo, hi, w, st = gpu_mst(X, 5, stats=True)
    say("scanned", st["scanned"])
    check_mst(X, 5, lo, hi, w)


def test_mst_small_sizes():
    for n in (2, 3, 17, 64, 65):
        X = datagen.random_uniform(n, 7, seed=n)
        ms = min(3, n - 1)
        say("mst n=%d" % n)
        lo, hi, w = gpu_mst(X, ms)
        check_tree_shape(n, lo, hi, w)
        check_mst(X, ms, lo, hi, w)


def test_mst_repeatable():
    X = datagen.spike_clips(5000, 15, seed=8)
    say("mst repeatable")
    a = gpu_mst(X, 10)
    b = gpu_mst(X, 10)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
