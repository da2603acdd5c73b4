"""GPU parity at the full workload sizes, in the configuration the benchmark runs.

* The two section workloads: every one of the 50,000 rows of the Kilosort4
  section against the oracle; on the wide section (63 row chunks) the rows on
  both sides of every chunk boundary, the whole short last chunk and a random
  sample.
* Clips 100,000 and 500,000: the oracle's core distances and its minimum
  spanning tree are stored (tests/golden/<workload>_oracle_tree.npz, written by
  tests/golden/make_golden.py from the oracle alone, since dense Prim over
  500,000 points takes hours on the host).  Every GPU core distance is checked
  against the oracle's at 1e-5 relative; every GPU tree edge's weight against
  its float64 weight; the sorted weight multisets and the total weight at 1e-5
  relative; and every GPU edge that the oracle's tree lacks must be a near-tie
  swap (the "HDBSCAN" page, "A lesson about tests: ties": where two edges are
  equally light either tree is correct).
* The HDBSCAN tail of the library on the GPU's tree against the oracle's tail
  on the same tree, exactly, and in summary against the oracle's tail on the
  oracle's own tree.
"""
import json
import os

import numpy as np
import pytest

import exact_knn_hdbscan_amd as ekh
from exact_knn_hdbscan_amd import datagen
from gpu_util import dev, host, say
from parity import (REL_D, REL_GAP, check_core, check_core_against, check_knn, compare_trees, dist_floor,
                    floor_sq, sq_norms)
from oracle import hdbscan_tail as otail
from test_hdbscan_tail import assert_same
from treecheck import PathMax

pytestmark = [pytest.mark.gpu, pytest.mark.fullsize]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_cache = {}


def workload(name):
    if name not in _cache:
        _cache.clear()
        _cache[name] = datagen.make(name)
    return _cache[name]


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.choice(n, k, replace=False)]))
    return rows


def knn_properties(idx, dist, m):
    assert idx.min() >= 0 and idx.max() < m
    srt = np.sort(idx, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])
    assert np.all(np.diff(dist, axis=1) >= 0), "rows must ascend"


def test_knn_ks4_section_every_row():
    """All 50,000 rows of the Kilosort4 section (k = 10 among the 5,000-point subset)."""
    wl = workload("ks4_section_50000x102")
    X, Y, k = wl["X"], wl["Y"], wl["k"]
    say("knn ks4_section_50000x102 full size, every row")
    i, dd = ekh.knn(dev(X), dev(Y), k)
    i, dd = host(i), host(dd)
    knn_properties(i, dd, Y.shape[1])
    rep = {}
    check_knn(X, Y, k, i, dd, report=rep, rescored=True)
    say("report", rep)
    assert rep["rows"] == X.shape[1]
    # subset members (every 10th point) find themselves first
    assert (i[::10, 0] == np.arange(Y.shape[1])).mean() > 0.99


def test_knn_wide_section_chunk_boundaries():
    """The wide section in row chunks of max_chunk_dots / m rows: the rows on
    both sides of every chunk boundary, every row of the short last chunk, and
    300 random rows."""
    wl = workload("wide_section_200000x200")
    X, Y, k = wl["X"], wl["Y"], wl["k"]
    n, m, d = X.shape[1], Y.shape[1], X.shape[0]
    dots = wl["max_chunk_bytes"] // 4
    plan = ekh.knn_plan(n, m, d, k, dots)
    cr = plan["chunk_rows"]
    starts = np.arange(0, n, cr)
    say("knn wide_section_200000x200 full size: %d chunks of %d rows, last %d rows (plan %s)"
        % (len(starts), cr, n - starts[-1], plan))
    assert len(starts) > 2 and n % cr != 0
    i, dd = ekh.knn(dev(X), dev(Y), k, max_chunk_dots=dots)
    i, dd = host(i), host(dd)
    knn_properties(i, dd, m)
    edge = np.concatenate([starts - 2, starts - 1, starts, starts + 1])
    last = np.arange(starts[-1], n)
    rows = np.unique(np.concatenate([edge[(edge >= 0) & (edge < n)], last, sample_rows(n, 300, 1)]))
    rep = {}
    check_knn(X, Y, k, i[rows], dd[rows], rows=rows, report=rep, rescored=True)
    say("report", rep)
    assert (i[::10, 0] == np.arange(m)).mean() > 0.99


def test_knn_section_reverse_orientation():
    """The other reading of 'neighbours of every point in Y': Y queries X (all 5,000 rows)."""
    wl = workload("ks4_section_50000x102")
    X, Y = wl["X"], wl["Y"]
    say("knn reverse orientation 5000 x 50000, every row")
    i, dd = ekh.knn(dev(Y), dev(X), 10)
    i, dd = host(i), host(dd)
    knn_properties(i, dd, X.shape[1])
    rep = {}
    check_knn(Y, X, 10, i, dd, report=rep, rescored=True)
    say("report", rep)


def _golden(name):
    path = os.path.join(GOLDEN, name + "_oracle.json")
    if not os.path.exists(path):
        pytest.skip("no stored oracle summary for " + name)
    return json.load(open(path))


def _golden_tree(name):
    path = os.path.join(GOLDEN, name + "_oracle_tree.npz")
    if not os.path.exists(path):
        pytest.skip("no stored oracle tree for " + name)
    with np.load(path) as z:
        return z["core"], z["lo"], z["hi"]


@pytest.mark.parametrize("name", ["clips_100000x61", "clips_500000x61"])
def test_core_and_mst_clips_full_size(name):
    wl = workload(name)
    X, ms = wl["X"], wl["min_samples"]
    d, n = X.shape
    g = _golden(name)
    ocore, olo, ohi = _golden_tree(name)
    assert g["n"] == n and g["min_samples"] == ms and ocore.shape == (n,) and olo.shape == (n - 1,)
    say("core + mst %s full size" % name)
    Xg = dev(X)
    core, ni, nd2 = ekh.core_distances(Xg, ms, return_neighbours=True)
    lo, hi, w, st = ekh.mst_boruvka(Xg, core, ms, ni, nd2, return_stats=True)
    core, ni, nd2 = host(core).astype(np.float64), host(ni), host(nd2)
    lo, hi, w = host(lo).astype(np.int64), host(hi).astype(np.int64), host(w).astype(np.float64)
    say("rounds %d scanned %s, of them against the largest component's complement %s"
        % (st["rounds"], st["scanned"], st["scanned_giant"]))
    assert st["rounds"] <= int(np.ceil(np.log2(n)))

    # every core distance against the oracle's (1e-5 relative; the floor only near 0)
    rep = {}
    check_core_against(X, core, ocore, report=rep)
    say("core", rep)
    assert rep["max_rel_core"] <= REL_D and rep["core_floor_used"] == 0
    assert abs(core.sum() - g["core_sum"]) <= REL_D * g["core_sum"]

    # sampled rows: whole neighbour lists against the oracle
    rows = sample_rows(n, 200, 3)
    rep_l = {}
    check_knn(X, X, ms + 1, ni[rows], np.sqrt(nd2[rows]), rows=rows, report=rep_l, gemm_lists=True)
    say("lists", rep_l)

    # the tree, edge by edge, against the oracle's
    rep_t = {}
    compare_trees(X, ocore, lo, hi, w, olo, ohi, report=rep_t)
    say("tree", rep_t)
    assert rep_t["rel_total"] <= REL_D and rep_t["max_rel_w"] <= REL_D and rep_t["w_floor_used"] == 0
    # the stored summary was written from the same oracle run
    assert abs(rep_t["total_oracle"] - g["mst_total_weight"]) <= 1e-12 * g["mst_total_weight"]

    # cycle property on sampled non-tree pairs of the GPU's own tree: neighbour
    # pairs of sampled points and random pairs, float64 weights from the oracle's cores
    from oracle import pair_weights
    rng = np.random.default_rng(4)
    a_s = rng.choice(n, 3000, replace=False)
    pa = np.concatenate([np.repeat(a_s, ms + 1), rng.integers(0, n, 20000)])
    pb = np.concatenate([ni[a_s].reshape(-1), rng.integers(0, n, 20000)])
    keep = pa != pb
    pa, pb = pa[keep], pb[keep]
    w_pair, _ = pair_weights(X, ocore, pa.astype(np.int32), pb.astype(np.int32))
    pm = PathMax(n, lo, hi)
    pmax = w[pm.query(pa, pb)]
    nx = sq_norms(X)
    eps_p = dist_floor(floor_sq(nx[pa], nx[pb]), w_pair, pmax)
    viol = w_pair < (1 - REL_GAP) * pmax - eps_p
    assert not viol.any(), "%d sampled pairs lighter than their tree path" % viol.sum()


@pytest.mark.parametrize("name", ["clips_100000x61", "clips_500000x61"])
def test_hdbscan_tail_clips_full_size(name):
    """Core distances and tree on the GPU, then the tail (min_cluster_size 20, the
    page's setting): exactly the oracle's tail on the same tree; and close to the
    oracle's tail on the oracle's own tree, which may differ where the two trees
    take different, equally light edges (the page's "ties" section)."""
    wl = workload(name)
    X, ms = wl["X"], wl["min_samples"]
    n = X.shape[1]
    say("tail %s full size" % name)
    Xg = dev(X)
    core, ni, nd2 = ekh.core_distances(Xg, ms, return_neighbours=True)
    lo, hi, w = ekh.mst_boruvka(Xg, core, ms, ni, nd2)
    lo, hi, w = host(lo), host(hi), host(w)
    labels, tree = ekh.hdbscan_tail(lo, hi, w, 20, return_tree=True)
    ref = otail.hdbscan_tail(lo.astype(np.int64), hi.astype(np.int64), w.astype(np.float64), n, 20)
    assert_same(labels, tree, ref, n)
    sizes = np.sort(np.bincount(labels[labels >= 0]))
    noise = int((labels < 0).sum())
    say("clusters %d noise %d sizes %s" % (len(sizes), noise, sizes.tolist()[:8]))
    assert len(sizes) >= 2
    g = _golden(name)
    gs = np.array(g["hdbscan_cluster_sizes_sorted"])
    say("oracle tree: clusters %d noise %d sizes %s" % (len(gs), g["hdbscan_noise"], gs.tolist()[:8]))
    assert len(sizes) == g["hdbscan_n_clusters"]
    tol = max(20, int(2e-3 * n))
    assert abs(noise - g["hdbscan_noise"]) <= tol
    assert np.abs(sizes - gs).max() <= tol


def test_mst_tiny_workload_matches_prim():
    """The tiny workload end to end against the oracle's Prim tree."""
    from parity import check_mst
    wl = workload("tiny_2000x60")
    X, ms = wl["X"], wl["min_samples"]
    say("tiny workload full path")
    Xg = dev(X)
    core, ni, nd2 = ekh.core_distances(Xg, ms, return_neighbours=True)
    lo, hi, w = ekh.mst_boruvka(Xg, core, ms, ni, nd2)
    rep = {}
    check_core(X, ms, host(core), report=rep)
    check_mst(X, ms, host(lo), host(hi), host(w), report=rep)
    say("report", rep)
    assert rep["max_rel_core"] <= REL_D and rep["rel_total"] <= REL_D
