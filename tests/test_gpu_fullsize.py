"""GPU parity at the full workload sizes, in the configuration the benchmark runs.

The oracle cannot run the whole 500,000-point problem inside a test, so each
check is one of:
  * sampled rows: kNN lists and core distances of a few hundred rows against
    the oracle's, computed one row at a time;
  * properties that hold at any size: a spanning tree with n - 1 edges, sorted
    by (w, lo, hi); every edge's distance against float64; the cycle property
    on sampled non-tree pairs (a pair's weight is never below the heaviest tree
    edge on the path between its ends, up to the near-tie tolerance);
  * stored oracle summaries (tests/golden/*_oracle.json, written by
    tests/golden/make_golden.py from the oracle alone): total tree weight and
    weight quantiles, core-distance sum and quantiles, and the HDBSCAN tail's
    cluster count, noise count and cluster sizes on the oracle's own tree;
  * the HDBSCAN tail of the library on the GPU's tree against the oracle's tail
    on the same tree, exactly (the oracle's tail is linear and runs in seconds).
"""
import json
import os

import numpy as np
import pytest
import torch

import exact_knn_hdbscan_amd as ekh
import oracle
from exact_knn_hdbscan_amd import datagen
from gpu_util import dev, host, say
from parity import REL_D, REL_GAP, check_core, check_knn, check_tree_shape, dist_floor, floor_sq, sq_norms
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


@pytest.mark.parametrize("name", ["ks4_section_50000x102", "wide_section_200000x200"])
def test_knn_sections_full_size(name):
    wl = workload(name)
    X, Y, k = wl["X"], wl["Y"], wl["k"]
    dots = wl.get("max_chunk_bytes", 0) // 4
    say("knn %s full size, max_chunk_dots=%d" % (name, dots))
    i, dd = ekh.knn(dev(X), dev(Y), k, max_chunk_dots=dots)
    i, dd = host(i), host(dd)
    knn_properties(i, dd, Y.shape[1])
    rows = sample_rows(X.shape[1], 300, 1)
    rep = {}
    check_knn(X, Y, k, i[rows], dd[rows], rows=rows, report=rep, rescored=True)
    say("report", rep)
    # subset members (every 10th point) find themselves first, within the floor
    own = i[::10, 0] == np.arange(Y.shape[1])
    assert own.mean() > 0.99


def test_knn_section_reverse_orientation():
    """The other reading of 'neighbours of every point in Y': Y queries X."""
    wl = workload("ks4_section_50000x102")
    X, Y = wl["X"], wl["Y"]
    say("knn reverse orientation 5000 x 50000")
    i, dd = ekh.knn(dev(Y), dev(X), 10)
    i, dd = host(i), host(dd)
    knn_properties(i, dd, X.shape[1])
    rows = sample_rows(Y.shape[1], 300, 2)
    check_knn(Y, X, 10, i[rows], dd[rows], rows=rows, rescored=True)


def _golden(name):
    path = os.path.join(GOLDEN, name + "_oracle.json")
    if not os.path.exists(path):
        pytest.skip("no stored oracle summary for " + name)
    return json.load(open(path))


@pytest.mark.parametrize("name", ["clips_100000x61", "clips_500000x61"])
def test_core_and_mst_clips_full_size(name):
    wl = workload(name)
    X, ms = wl["X"], wl["min_samples"]
    d, n = X.shape
    say("core + mst %s full size" % name)
    Xg = dev(X)
    core, ni, nd2 = ekh.core_distances(Xg, ms, return_neighbours=True)
    lo, hi, w, st = ekh.mst_boruvka(Xg, core, ms, ni, nd2, return_stats=True)
    core, ni, nd2 = host(core).astype(np.float64), host(ni), host(nd2)
    lo, hi, w = host(lo).astype(np.int64), host(hi).astype(np.int64), host(w).astype(np.float64)
    say("rounds %d scanned %s, of them against the largest component's complement %s"
        % (st["rounds"], st["scanned"], st["scanned_giant"]))
    assert st["rounds"] <= int(np.ceil(np.log2(n)))
    # the last round's largest component (most of the points) takes the complement scan
    assert sum(st["scanned_giant"]) > 0

    # sampled rows: lists and core distances against the oracle
    rows = sample_rows(n, 200, 3)
    check_knn(X, X, ms + 1, ni[rows], np.sqrt(nd2[rows]), rows=rows)
    check_core(X, ms, core[rows], rows=rows)

    # the tree at full size
    check_tree_shape(n, lo, hi, w)
    nx = sq_norms(X)
    # every edge: the GPU weight is max(core_lo, core_hi, D) with D against float64
    dist64 = np.sqrt(np.maximum(((X[:, lo].astype(np.float64) - X[:, hi].astype(np.float64)) ** 2).sum(0), 0))
    w_expect = np.maximum(np.maximum(core[lo], core[hi]), dist64)
    eps_w = dist_floor(floor_sq(d, nx[lo], nx[hi]), w, w_expect)
    bad = np.abs(w - w_expect) > REL_D * w_expect + eps_w
    assert not bad.any(), "%d edges whose weight does not match their endpoints" % bad.sum()

    # cycle property on sampled non-tree pairs: neighbour pairs of sampled points and random pairs
    rng = np.random.default_rng(4)
    a_s = rng.choice(n, 3000, replace=False)
    pa = np.concatenate([np.repeat(a_s, ms + 1), rng.integers(0, n, 20000)])
    pb = np.concatenate([ni[a_s].reshape(-1), rng.integers(0, n, 20000)])
    keep = pa != pb
    pa, pb = pa[keep], pb[keep]
    # pair weights from float64 distances and the GPU core distances (those are
    # checked against the oracle on the sampled rows above)
    dpair = np.sqrt(((X[:, pa].astype(np.float64) - X[:, pb].astype(np.float64)) ** 2).sum(0))
    w_pair = np.maximum(np.maximum(core[pa], core[pb]), dpair)
    pm = PathMax(n, lo, hi)
    pmax = w[pm.query(pa, pb)]
    eps_p = dist_floor(floor_sq(d, nx[pa], nx[pb]) + floor_sq(d, nx.max(), nx.max()), w_pair, pmax)
    viol = w_pair < (1 - REL_GAP) * pmax - eps_p
    assert not viol.any(), "%d sampled pairs lighter than their tree path" % viol.sum()

    # stored oracle summaries
    g = _golden(name)
    assert g["n"] == n and g["min_samples"] == ms
    tol_total = REL_D * g["mst_total_weight"] + eps_w.sum()
    say("total weight gpu %.9g oracle %.9g (diff %.3g, tol %.3g)" % (w.sum(), g["mst_total_weight"],
                                                                   w.sum() - g["mst_total_weight"], tol_total))
    assert abs(w.sum() - g["mst_total_weight"]) <= tol_total
    qs = np.quantile(w, g["quantile_levels"])
    np.testing.assert_allclose(qs, g["mst_weight_quantiles"], rtol=1e-4, atol=float(eps_w.max()))
    cq = np.quantile(core, g["quantile_levels"])
    np.testing.assert_allclose(cq, g["core_quantiles"], rtol=1e-4, atol=1e-4)
    eps_core = dist_floor(floor_sq(d, nx, nx.max()), core, core)
    assert abs(core.sum() - g["core_sum"]) <= REL_D * g["core_sum"] + eps_core.sum()


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
    if "hdbscan_n_clusters" not in g:
        pytest.skip("stored oracle summary has no tail figures")
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
    check_core(X, ms, host(core))
    check_mst(X, ms, host(lo), host(hi), host(w))
