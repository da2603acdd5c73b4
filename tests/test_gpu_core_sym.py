"""The symmetric self-kNN of ekh_core_distances (every pair computed once, the
column side through per-point candidate buffers) against the path that
computes every pair from both sides (EKH_CORE_DENSE=1): the same core
distances and neighbour rows, bit for bit.  Parity of both with the oracle is
in the other GPU tests (the symmetric path runs from 16,384 points on)."""
import os

import numpy as np
import pytest

import exact_knn_hdbscan_amd as ekh
from exact_knn_hdbscan_amd import datagen
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def run_both(X, ms, ld=None):
    Xg = dev(X, ld=ld)
    os.environ["EKH_CORE_DENSE"] = "1"
    try:
        c0, i0, d0 = ekh.core_distances(Xg, ms, return_neighbours=True)
        c0, i0, d0 = host(c0), host(i0), host(d0)
    finally:
        del os.environ["EKH_CORE_DENSE"]
    c1, i1, d1 = ekh.core_distances(Xg, ms, return_neighbours=True)
    return (c0, i0, d0), (host(c1), host(i1), host(d1))


def assert_same(a, b):
    (c0, i0, d0), (c1, i1, d1) = a, b
    assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32)), "core distances differ"
    bad = np.nonzero((i0 != i1).any(axis=1))[0]
    assert bad.size == 0, "rows %s differ: %s vs %s" % (bad[:5].tolist(), i0[bad[:2]].tolist(), i1[bad[:2]].tolist())
    assert np.array_equal(d0.view(np.uint32), d1.view(np.uint32)), "squared distances differ"


@pytest.mark.parametrize("n,d,ms,seed", [
    (16384, 61, 10, 1),   # the smallest size that takes the symmetric path, whole tiles
    (40001, 61, 10, 2),   # a partial last query tile and database tile
    (20000, 16, 5, 3),    # list length 8 (k = 6), 4 k-steps
    (23457, 7, 15, 4),    # list length 16, 2 k-steps, one column block per wave
    (17000, 33, 31, 5),   # list length 32
    (30000, 64, 1, 6),    # min_samples 1 (core 0, lists of 2)
])
def test_core_symmetric_equals_dense(n, d, ms, seed):
    X = datagen.gaussian_mixture(n, d, 30, seed=seed)
    say("core symmetric vs dense n=%d d=%d ms=%d" % (n, d, ms))
    assert_same(*run_both(X, ms))


def _random_shapes(count, seed):
    # seeded draws over the symmetric path's range: n from its threshold to 60,000 (whole and partial
    # tiles), every d up to 64 (odd feature counts, partial k-steps), min_samples 1 to 31 (every list length)
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(16384, 60001)), int(rng.integers(1, 65)), int(rng.integers(1, 32)), int(rng.integers(0, 1 << 20)))
            for _ in range(count)]


@pytest.mark.parametrize("n,d,ms,seed", _random_shapes(8, 2026))
def test_core_symmetric_equals_dense_random_shapes(n, d, ms, seed):
    X = datagen.gaussian_mixture(n, d, 40, seed=seed)
    say("core symmetric vs dense (random shape) n=%d d=%d ms=%d seed=%d" % (n, d, ms, seed))
    assert_same(*run_both(X, ms))


@pytest.mark.parametrize("n,d,ms,ld", [
    (16385, 1, 10, None),      # d = 1; the last query tile holds one point, the last database tile one row
    (18000, 61, 10, 18013),    # leading dimension past n
    (16512, 64, 16, None),     # exactly 129 query tiles, list length 32 (k = 17)
])
def test_core_symmetric_edge_shapes(n, d, ms, ld):
    X = datagen.gaussian_mixture(n, d, 25, seed=n % 31)
    say("core symmetric vs dense n=%d d=%d ms=%d ld=%s" % (n, d, ms, ld))
    assert_same(*run_both(X, ms, ld))


def test_core_symmetric_clips_100000():
    X = datagen.make("clips_100000x61")["X"]
    say("core symmetric vs dense: clips 100,000 x 61")
    assert_same(*run_both(X, 10))


def test_core_symmetric_duplicate_groups_overflow():
    """80 points, each repeated 300 times: every D2 within a group is exactly 0,
    so each point has up to 299 column candidates at its bound, more than a
    buffer holds; those query tiles are recomputed by the dense kernel, and
    the index order decides every tie alike."""
    base = datagen.gaussian_mixture(80, 12, 8, seed=7)
    X = np.repeat(base, 300, axis=1)
    say("core symmetric vs dense: 80 groups of 300 duplicates (buffer overflow)")
    a, b = run_both(X, 10)
    assert_same(a, b)
    # every D2 in a list is 0, so each point's list is the 11 lowest indices of its group
    c1, i1, _ = b
    assert np.all(c1 == 0)
    g0 = (np.arange(X.shape[1]) // 300) * 300
    assert np.array_equal(i1, g0[:, None] + np.arange(11)[None, :])


def test_core_symmetric_shuffled_duplicates():
    """The same groups in random order (candidates of a group spread over every query tile)."""
    rng = np.random.default_rng(9)
    base = datagen.gaussian_mixture(80, 12, 8, seed=7)
    X = np.ascontiguousarray(np.repeat(base, 300, axis=1)[:, rng.permutation(24000)])
    say("core symmetric vs dense: shuffled duplicate groups")
    assert_same(*run_both(X, 10))
