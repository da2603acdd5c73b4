"""GPU parity of ekh_knn / ekh_core_distances against the float64 oracle."""
import numpy as np
import pytest

import exact_knn_hdbscan_amd as ekh
import oracle
from exact_knn_hdbscan_amd import datagen
from gpu_util import dev, host, say
from parity import REL_D, check_core, check_knn

pytestmark = pytest.mark.gpu


def test_knn_tiny_self():
    X = datagen.make("tiny_2000x60")["X"]
    say("knn tiny 2000x60 k=10, X and Y separate copies")
    i, dd = ekh.knn(dev(X), dev(X), 10)
    check_knn(X, X, 10, host(i), host(dd), rescored=True)
    say("knn tiny 2000x60 self k=10")
    # the same tensor as X and Y makes the set its own database
    Xg = dev(X)
    i, dd = ekh.knn(Xg, Xg, 10)
    rep = {}
    check_knn(X, X, 10, host(i), host(dd), report=rep, rescored=True)
    say("report", rep)
    assert np.all(host(i)[:, 0] == np.arange(2000))
    assert np.all(host(dd)[:, 0] == 0)


def test_knn_odd_sizes_and_leading_dimension():
    rng = np.random.default_rng(5)
    X = datagen.gaussian_mixture(2001, 61, 7, seed=1)
    Y = datagen.gaussian_mixture(777, 61, 7, seed=2)
    say("knn odd n=2001 m=777 d=61 ld padded")
    i, dd = ekh.knn(dev(X, ld=2011), dev(Y, ld=781), 10)
    check_knn(X, Y, 10, host(i), host(dd), rescored=True)


def test_knn_caller_outputs_and_workspace():
    """Outputs and workspace passed in: the same lists bit for bit; a workspace
    below the size the library needs is refused."""
    import torch
    X = datagen.gaussian_mixture(3001, 61, 6, seed=21)
    Y = datagen.gaussian_mixture(1499, 61, 6, seed=22)
    Xg, Yg = dev(X), dev(Y)
    say("knn with caller outputs and workspace")
    i0, d0 = ekh.knn(Xg, Yg, 9)
    need = ekh.knn_workspace_bytes(3001, 1499, 61, 9)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    oi = torch.full((3001, 9), -7, dtype=torch.int32, device="cuda:0")
    od = torch.full((3001, 9), -7.0, dtype=torch.float32, device="cuda:0")
    i1, d1 = ekh.knn(Xg, Yg, 9, workspace=ws, out_idx=oi, out_dist=od)
    assert i1.data_ptr() == oi.data_ptr() and d1.data_ptr() == od.data_ptr()
    assert np.array_equal(host(i0), host(i1)) and np.array_equal(host(d0).view(np.uint32), host(d1).view(np.uint32))
    with pytest.raises(ekh.EkhError):
        ekh.knn(Xg, Yg, 9, workspace=ws[: need - 1])
    with pytest.raises(ValueError):
        ekh.knn(Xg, Yg, 9, out_idx=oi[:, :8])


def test_knn_and_core_leading_dimension_past_2_25():
    """A leading dimension of 2^25 + 17 floats (the tiles read the point-major
    copy, so no tile address depends on it): ekh_knn and ekh_core_distances."""
    ld = (1 << 25) + 17
    X = datagen.gaussian_mixture(1500, 3, 4, seed=11)
    Y = datagen.gaussian_mixture(1201, 3, 4, seed=12)
    say("knn and core, d=3, ld = 2^25 + 17")
    i, dd = ekh.knn(dev(X, ld=ld), dev(Y, ld=ld), 7)
    check_knn(X, Y, 7, host(i), host(dd), rescored=True)
    rep = {}
    core = ekh.core_distances(dev(X, ld=ld), 5)
    check_core(X, 5, host(core), report=rep)
    assert rep["max_rel_core"] <= REL_D


# every tile-kernel instantiation (QM = 4 ceil(d / 16) k-steps: 4, 8, ..., 64),
# at both ends of its range where it matters
@pytest.mark.parametrize("d", [1, 3, 16, 17, 33, 48, 60, 64, 65, 90, 102, 112, 128, 129, 150, 170, 185, 200, 220,
                               225, 240, 256])
def test_knn_dimensions(d):
    X = datagen.gaussian_mixture(333, d, 5, seed=d)
    Y = datagen.gaussian_mixture(517, d, 5, seed=d + 1000)
    say("knn d=%d" % d)
    i, dd = ekh.knn(dev(X), dev(Y), 10)
    check_knn(X, Y, 10, host(i), host(dd), rescored=True)


@pytest.mark.parametrize("k,d", [(2, 33), (4, 90), (8, 150), (16, 102), (32, 200), (32, 250)])
def test_knn_k_values_other_widths(k, d):
    """List lengths other than K = 11 at other tile-kernel widths."""
    X = datagen.gaussian_mixture(900, d, 6, seed=k + d)
    say("knn self k=%d d=%d" % (k, d))
    Xg = dev(X)
    i, dd = ekh.knn(Xg, Xg, k)
    check_knn(X, X, k, host(i), host(dd), rescored=True)


@pytest.mark.parametrize("k", [1, 2, 3, 8, 10, 11, 12, 16, 17, 32])
def test_knn_k_values(k):
    X = datagen.spike_clips(700, 5, seed=k)
    say("knn self k=%d" % k)
    Xg = dev(X)
    i, dd = ekh.knn(Xg, Xg, k)
    check_knn(X, X, k, host(i), host(dd), rescored=True)


@pytest.mark.parametrize("d", [5, 61, 100, 200])
def test_knn_integer_grid_exact(d):
    """Integer coordinates: every D2 is exact in float32, so indices (ties in
    ascending order) and distances must equal the oracle's exactly."""
    X = datagen.integer_grid(600, d, seed=d, half_range=2)
    Y = datagen.integer_grid(450, d, seed=d + 7, half_range=2)
    for self_ in (True, False):
        say("knn integer d=%d self=%s" % (d, self_))
        if self_:
            Xg = dev(X)
            i, dd = ekh.knn(Xg, Xg, 16)
            oi, od2 = oracle.knn(X, X, 16)
        else:
            i, dd = ekh.knn(dev(X), dev(Y), 16)
            oi, od2 = oracle.knn(X, Y, 16)
        np.testing.assert_array_equal(host(i), oi)
        np.testing.assert_array_equal(host(dd), np.sqrt(od2.astype(np.float32)))
        assert np.any(od2[:, 1:] == od2[:, :-1])


@pytest.mark.parametrize("d", [7, 61])
def test_knn_short_databases_every_tile_count(d):
    """Databases of 1 to 5 tiles of 32 rows (full and partial last tiles): at
    d <= 64 the tile loop takes a barrier after every second tile with four
    buffers, so odd and even tile counts and a lone partial tile take
    different paths through it."""
    X = datagen.gaussian_mixture(700, d, 5, seed=d)
    for m in (1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 129, 160):
        Y = datagen.gaussian_mixture(m, d, 3, seed=m)
        k = min(10, m)
        say("knn n=700 m=%d d=%d k=%d" % (m, d, k))
        i, dd = ekh.knn(dev(X), dev(Y), k)
        check_knn(X, Y, k, host(i), host(dd), rescored=True)


def test_knn_k_equals_m_and_n():
    X = datagen.random_uniform(31, 9, seed=3)
    Y = datagen.random_uniform(20, 9, seed=4)
    say("knn k = m")
    i, dd = ekh.knn(dev(X), dev(Y), 20)
    check_knn(X, Y, 20, host(i), host(dd), rescored=True)
    assert all(sorted(r) == list(range(20)) for r in host(i).tolist())
    Xg = dev(X)
    i, dd = ekh.knn(Xg, Xg, 31)
    check_knn(X, X, 31, host(i), host(dd), rescored=True)


def test_knn_duplicates():
    X = datagen.duplicates(9, 61, seed=3, n_other=300)
    say("knn duplicates")
    Xg = dev(X)
    i, dd = ekh.knn(Xg, Xg, 12)
    hi = host(i)
    check_knn(X, X, 12, hi, host(dd), rescored=True)
    for r in range(9):
        assert sorted(hi[r, :9].tolist()) == list(range(9))


def test_knn_chunk_and_split_invariance():
    X = datagen.gaussian_mixture(5000, 102, 20, seed=11)
    Y = datagen.every_kth(X, 2)
    Xg, Yg = dev(X), dev(Y)
    say("knn chunking invariance")
    ref_i, ref_d = ekh.knn(Xg, Yg, 10)
    ref_i, ref_d = host(ref_i), host(ref_d)
    check_knn(X, Y, 10, ref_i, ref_d, rescored=True)
    for dots in (1, 2500 * 128, 2500 * 1000, 2500 * 4096):
        i, dd = ekh.knn(Xg, Yg, 10, max_chunk_dots=dots)
        np.testing.assert_array_equal(host(i), ref_i)
        np.testing.assert_array_equal(host(dd), ref_d)


@pytest.mark.parametrize("n,m,d,k,dots,layout", [
    # 813 query tiles of 64 rows (d = 102), 768 resident: one whole round, 45 split tiles
    (52001, 3001, 102, 10, 0, (768, 0)),
    # 774 tiles of 128 rows (d = 61, K = 11): one whole round, 6 split tiles (ragged last tile)
    (99001, 1500, 61, 11, 0, (768, 0)),
    # two chunks: 99,968 rows (781 tiles: one whole round + 13 split tiles), then 20,032 rows (all split)
    (120000, 1000, 16, 8, 100_000_000, (768, 0)),
    # K = 32 lists: two workgroups per CU (512 resident), 648 tiles of 64 rows: 512 whole + 136 split
    (41435, 2552, 128, 21, 0, (512, 0)),
])
def test_knn_whole_round_and_split_tail(n, m, d, k, dots, layout):
    """The launch layout with whole tiles for the full rounds of resident
    workgroups and database splits for the rest: parity with the oracle on every
    row, and bitwise the same result as the layout with every tile split alike
    (chunks of fewer tiles than one round)."""
    p = ekh.knn_plan(n, m, d, k, dots)
    assert (p["body_tiles"], p["last_body_tiles"] if dots else 0) == layout and p["splits"] > 1, p
    X = datagen.gaussian_mixture(n, d, 20, seed=n % 97)
    Y = datagen.gaussian_mixture(m, d, 20, seed=m % 89)
    Xg, Yg = dev(X), dev(Y)
    say("knn n=%d m=%d d=%d k=%d dots=%d plan %s" % (n, m, d, k, dots, p))
    i, dd = ekh.knn(Xg, Yg, k, max_chunk_dots=dots)
    i, dd = host(i), host(dd)
    check_knn(X, Y, k, i, dd, rescored=True)
    small = 64 * p["tile_rows"] * m  # 64 tiles per chunk: fewer than one round of a chunk's share
    q = ekh.knn_plan(n, m, d, k, small)
    assert q["body_tiles"] == 0 and q["last_body_tiles"] == 0, q
    i2, d2 = ekh.knn(Xg, Yg, k, max_chunk_dots=small)
    np.testing.assert_array_equal(host(i2), i)
    np.testing.assert_array_equal(host(d2), dd)


def test_knn_query_tiles_fill_whole_rounds():
    """98,304 queries = 768 tiles of 128 rows, exactly one round of resident
    workgroups: no split tail, every tile reads the whole database."""
    n, m, d, k = 98304, 1000, 61, 11
    p = ekh.knn_plan(n, m, d, k)
    assert p["body_tiles"] == 0 and p["splits"] == 1, p
    X = datagen.gaussian_mixture(n, d, 15, seed=21)
    Y = datagen.gaussian_mixture(m, d, 15, seed=22)
    say("knn n=%d m=%d: %s" % (n, m, p))
    i, dd = ekh.knn(dev(X), dev(Y), k)
    check_knn(X, Y, k, host(i), host(dd), rescored=True)


def test_knn_few_queries_long_database():
    """200 queries against 2,000,000 points: two query tiles, so the database
    is split 384 ways (768 workgroups) and the merge combines 384 lists a row."""
    n, m, d, k = 200, 2_000_000, 16, 10
    p = ekh.knn_plan(n, m, d, k)
    assert p["splits"] > 64, p
    X = datagen.gaussian_mixture(n, d, 5, seed=31)
    Y = datagen.gaussian_mixture(m, d, 50, seed=32)
    say("knn n=%d m=%d: %s" % (n, m, p))
    i, dd = ekh.knn(dev(X), dev(Y), k)
    check_knn(X, Y, k, host(i), host(dd), rescored=True)


def test_knn_repeatable():
    X = datagen.spike_clips(3000, 8, seed=4)
    Xg = dev(X)
    say("knn repeatable")
    a = [tuple(host(t) for t in ekh.knn(Xg, Xg, 11)) for _ in range(3)]
    for i, dd in a[1:]:
        np.testing.assert_array_equal(i, a[0][0])
        np.testing.assert_array_equal(dd, a[0][1])


def test_squared_distance_symmetric_bitwise():
    """D2(a, b) == D2(b, a) bit for bit: required so that the list-based
    shortcuts and the scan agree on every edge weight."""
    X = datagen.spike_clips(32, 3, seed=21)
    say("symmetry")
    core, ni, nd2 = ekh.core_distances(dev(X), 31, return_neighbours=True)
    ni, nd2 = host(ni), host(nd2)
    M = np.full((32, 32), np.nan, np.float32)
    for a in range(32):
        M[a, ni[a]] = nd2[a]
    assert not np.isnan(M).any()
    np.testing.assert_array_equal(M, M.T)
    assert np.all(np.diag(M) == 0)


def test_core_tiny_and_lists():
    X = datagen.make("tiny_2000x60")["X"]
    say("core tiny ms=10")
    core, ni, nd2 = ekh.core_distances(dev(X), 10, return_neighbours=True)
    core, ni, nd2 = host(core), host(ni), host(nd2)
    rep = {}
    check_core(X, 10, core, report=rep)
    check_knn(X, X, 11, ni, np.sqrt(nd2), report=rep, gemm_lists=True)
    say("report", rep)
    # the core distance is the direct-difference distance of the 10th-nearest list
    # entry; the list's own D2 is the GEMM form, equal to it within float32 rounding
    from parity import true_sqdist
    t2 = np.sort(true_sqdist(X, np.arange(X.shape[1]), X, ni), axis=1)
    np.testing.assert_allclose(core.astype(np.float64), np.sqrt(t2[:, 9]), rtol=2e-6)
    np.testing.assert_allclose(core, np.sqrt(nd2[:, 9]), rtol=1e-5)


def test_core_closed_forms():
    X = datagen.collinear(101, 61, spacing=2.0)
    say("core collinear")
    Xg = dev(X)
    c = host(ekh.core_distances(Xg, 3))
    exp = np.full(101, 2.0, np.float32)
    exp[0] = exp[-1] = 4.0
    np.testing.assert_array_equal(c, exp)
    np.testing.assert_array_equal(host(ekh.core_distances(Xg, 1)), np.zeros(101, np.float32))
    D = datagen.duplicates(12, 61, seed=5, n_other=50)
    c = host(ekh.core_distances(dev(D), 10))
    assert np.all(c[:12] == 0) and np.all(c[12:] > 0)


def test_identical_points_at_distance_zero():
    """Norms come from the same MFMA contraction as the dot products, so two
    bitwise-identical points are at D2 = 0 exactly, wherever they sit."""
    rng = np.random.default_rng(12)
    base = datagen.spike_clips(900, 6, seed=12)
    X = base.copy()
    src = rng.choice(900, 60, replace=False)
    dst = rng.choice(np.setdiff1d(np.arange(900), src), 60, replace=False)
    X[:, dst] = X[:, src]
    say("identical points, scattered")
    Xg = dev(X)
    core, ni, nd2 = ekh.core_distances(Xg, 3, return_neighbours=True)
    ni, nd2 = host(ni), host(nd2)
    for a, b in zip(src, dst):
        for p, q in ((a, b), (b, a)):
            row = ni[p].tolist()
            assert q in row and nd2[p][row.index(q)] == 0.0
