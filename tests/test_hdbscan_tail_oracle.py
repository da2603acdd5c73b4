"""Pins of the oracle's HDBSCAN tail (oracle/hdbscan_tail.py), none taken from the oracle itself.

* closed forms: hand-built trees whose condensed tree, stabilities and
  selection are worked out by hand in exact binary fractions, including an
  exact excess-of-mass tie (the parent is kept) and the boundary
  size == min_cluster_size;
* scipy: every cluster of the condensed tree is a flat cluster of scipy's own
  single linkage over the mutual-reachability matrix, cut just below the
  cluster's birth distance;
* scikit-learn's HDBSCAN on blobs: the same partition into clusters and noise
  at every point not attached through a tie (an informal cross-check of the
  whole definition against a third-party implementation);
* invariants: every point is an entry exactly once, sizes add up, selected
  clusters are disjoint and hold >= min_cluster_size points.

The second half plants plausible mistakes in a copy of the module and requires
some pin to fail for each.
"""
import importlib.util
import os
import sys

import numpy as np
import pytest

import oracle
from oracle import hdbscan_tail as tail_mod

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _edges(lst):
    lo = np.array([min(a, b) for a, b, _ in lst], np.int64)
    hi = np.array([max(a, b) for a, b, _ in lst], np.int64)
    w = np.array([x for _, _, x in lst], np.float64)
    return lo, hi, w


# A = {0,1,2} and B = {3,4,5} (inner edges 0.5, joined at 1.0); six loose points
# hang off 0 and 3 at 2.0; Y = {12,13,14} (inner 0.5) joins at 4.0.
TIE_TREE = [(0, 1, 0.5), (1, 2, 0.5), (3, 4, 0.5), (4, 5, 0.5), (2, 3, 1.0),
            (0, 6, 2.0), (0, 7, 2.0), (0, 8, 2.0), (3, 9, 2.0), (3, 10, 2.0), (3, 11, 2.0),
            (12, 13, 0.5), (13, 14, 0.5), (5, 12, 4.0)]


def check_tie_tree_parent_kept(t):
    """min_cluster_size 3.  Root 15 -> X = {0..11} (16) and Y (17) at lambda 1/4;
    X sheds 6 loose points at 1/2 and splits at 1 into A (18), B (19), whose
    points leave at 2.  S(X) = 6 (1/2 - 1/4) + 6 (1 - 1/4) = 6 = S(A) + S(B)
    = 3 + 3: on the tie the parent is kept."""
    lo, hi, w = _edges(TIE_TREE)
    r = t.hdbscan_tail(lo, hi, w, 15, 3)
    st = r["stability"]
    assert r["birth"] == {15: 0.0, 16: 0.25, 17: 0.25, 18: 1.0, 19: 1.0}
    assert (st[16], st[17], st[18], st[19]) == (6.0, 5.25, 3.0, 3.0)
    assert st[15] == 15 * 0.25
    assert r["selected"] == [16, 17]
    assert list(r["labels"]) == [0] * 12 + [1] * 3
    ent = r["entries"]
    assert ent[:2] == [(15, 16, 0.25, 12), (15, 17, 0.25, 3)]
    assert sorted(e for e in ent if e[0] == 16 and e[1] < 15) == [(16, p, 0.5, 1) for p in range(6, 12)]
    assert [e for e in ent if e[0] == 16 and e[1] >= 15] == [(16, 18, 1.0, 3), (16, 19, 1.0, 3)]
    assert [e for e in ent if e[0] == 18] == [(18, p, 2.0, 1) for p in range(3)]


def check_tie_tree_boundary_size(t):
    """min_cluster_size 4: Y (3 points) leaves the root at 1/4; A and B are too
    small, so X sheds everything and the root never splits: all noise."""
    lo, hi, w = _edges(TIE_TREE)
    r = t.hdbscan_tail(lo, hi, w, 15, 4)
    assert r["selected"] == []
    assert list(r["birth"]) == [15]
    assert (r["labels"] == -1).all()
    lam = {e[1]: e[2] for e in r["entries"]}
    assert [lam[p] for p in range(15)] == [1.0] * 6 + [0.5] * 6 + [0.25] * 3


def check_line_groups_closed_form(t):
    """Two groups of 5 on a line, spacing 1 and 2, gap 10: two clusters born at
    1/10; S = 5 (1 - 1/10) = 4.5 and 5 (1/2 - 1/10) = 2.0."""
    lst = [(i, i + 1, 1.0) for i in range(4)] + [(4, 5, 10.0)] + [(i, i + 1, 2.0) for i in range(5, 9)]
    lo, hi, w = _edges(lst)
    r = t.hdbscan_tail(lo, hi, w, 10, 3)
    assert r["selected"] == [11, 12]
    assert r["stability"][11] == 5 * (1.0 - 0.1)
    assert r["stability"][12] == 5 * (0.5 - 0.1)
    assert list(r["labels"]) == [0] * 5 + [1] * 5
    r6 = t.hdbscan_tail(lo, hi, w, 10, 6)  # both groups below 6: all noise
    assert r6["selected"] == [] and (r6["labels"] == -1).all()


def check_nested_children_win(t):
    """AB = A {0..3} + B {4..7} (inner 1, joined at 2), C {8..11} (inner 1) at 22;
    min_cluster_size 4.  S(AB) = 8 (1/2 - 1/22) < S(A) + S(B) = 2 + 2, so A and B
    are chosen; with the A-B join at 1.25 the parent wins instead."""
    def tree(gap):
        return ([(i, i + 1, 1.0) for i in range(3)] + [(3, 4, gap)] + [(i, i + 1, 1.0) for i in range(4, 7)]
                + [(7, 8, 22.0)] + [(i, i + 1, 1.0) for i in range(8, 11)])
    lo, hi, w = _edges(tree(2.0))
    r = t.hdbscan_tail(lo, hi, w, 12, 4)
    # ids: root 12; AB 13, C 14 (born 1/22); A 15, B 16 (born 1/2)
    assert r["selected"] == [14, 15, 16]
    assert list(r["labels"]) == [1] * 4 + [2] * 4 + [0] * 4
    lo, hi, w = _edges(tree(1.25))
    r = t.hdbscan_tail(lo, hi, w, 12, 4)
    assert r["selected"] == [13, 14]
    assert list(r["labels"]) == [0] * 8 + [1] * 4


def check_zero_weights(t):
    """Duplicates: groups merging at w = 0 have lambda = inf.  Two groups of 3
    identical points joined at 1: each cluster's points leave at inf, so both
    clusters have infinite stability and are selected; a cluster born at inf
    has stability 0 (inf - inf terms count 0)."""
    lst = [(0, 1, 0.0), (1, 2, 0.0), (3, 4, 0.0), (4, 5, 0.0), (2, 3, 1.0)]
    lo, hi, w = _edges(lst)
    r = t.hdbscan_tail(lo, hi, w, 6, 3)
    assert r["selected"] == [7, 8]
    assert r["stability"][7] == np.inf
    assert list(r["labels"]) == [0, 0, 0, 1, 1, 1]
    # G1 = {0, 1, 5} and G2 = {2, 3, 4} at w = 0, joined by (4, 5) at w = 0, which
    # sorts after both groups' edges; point 6 hangs off at 1.  The root sheds 6
    # at lambda 1, then splits at w = 0 into two clusters born at inf.
    lst2 = [(0, 1, 0.0), (1, 5, 0.0), (2, 3, 0.0), (3, 4, 0.0), (4, 5, 0.0), (5, 6, 1.0)]
    lo, hi, w = _edges(lst2)
    r2 = t.hdbscan_tail(lo, hi, w, 7, 3)
    assert r2["birth"] == {7: 0.0, 8: np.inf, 9: np.inf}
    assert r2["stability"][8] == 0.0 and r2["stability"][7] == np.inf
    assert r2["selected"] == [8, 9]
    assert list(r2["labels"]) == [0, 0, 1, 1, 1, 0, -1]


def check_tie_order_decides_attachment(t):
    """X = {0..3} and Y = {4..7} (inner 0.5); point 8 hangs off X by (1, 8) and
    X meets Y by (3, 4), both at 1.0.  In (w, lo, hi) order (1, 8) merges first,
    so the top split at lambda 1 is (X + 8 | Y): clusters 10 = X + {8} and 11 = Y,
    and 8 leaves cluster 10 at its birth (it is a member).  Merging (3, 4) first
    would make 8 noise."""
    lst = [(0, 1, 0.5), (1, 2, 0.5), (2, 3, 0.5), (4, 5, 0.5), (5, 6, 0.5), (6, 7, 0.5),
           (1, 8, 1.0), (3, 4, 1.0)]
    lo, hi, w = _edges(lst)
    r = t.hdbscan_tail(lo, hi, w, 9, 3)
    assert r["birth"] == {9: 0.0, 10: 1.0, 11: 1.0}
    assert (r["stability"][10], r["stability"][11]) == (4.0, 4.0)
    assert (10, 8, 1.0, 1) in r["entries"]
    assert list(r["labels"]) == [0, 0, 0, 0, 1, 1, 1, 1, 0]


def _blobs(seed, n_per, centers, d, noise=0):
    rng = np.random.default_rng(seed)
    mu = rng.uniform(-10, 10, (centers, d))
    pts = [rng.normal(mu[c], rng.uniform(0.5, 1.5), (n_per, d)) for c in range(centers)]
    if noise:
        pts.append(rng.uniform(-14, 14, (noise, d)))
    X = np.concatenate(pts)
    X = X[rng.permutation(len(X))]
    return np.ascontiguousarray(X.T.astype(np.float32))


def _tree(X, ms):
    core = oracle.core_distances(X, ms)
    return oracle.mst_prim(X, core)


def check_clusters_are_scipy_single_linkage_cuts(t):
    from scipy.cluster.hierarchy import fcluster, linkage
    from scipy.spatial.distance import squareform
    X = _blobs(3, 60, 4, 5, noise=30)
    ms, mcs = 5, 10
    n = X.shape[1]
    core = oracle.core_distances(X, ms)
    lo, hi, w = oracle.mst_prim(X, core)
    r = t.hdbscan_tail(lo, hi, w, n, mcs)
    M = oracle.mutual_reachability_matrix(X, core)
    np.fill_diagonal(M, 0.0)
    Z = linkage(squareform(M, checks=False), method="single")
    members = {}
    parent_of = {e[1]: e[0] for e in r["entries"]}
    for p in range(n):
        c = parent_of[p]
        while c is not None:
            members.setdefault(c, set()).add(p)
            c = parent_of.get(c)
    assert len(r["birth"]) > 3
    for c, b in r["birth"].items():
        if c == n:
            continue
        cut = (1.0 / b) * (1 - 1e-9)
        flat = fcluster(Z, cut, criterion="distance")
        mem = sorted(members[c])
        assert len(set(flat[mem])) == 1, "cluster %d is split by the cut" % c
        assert (flat == flat[mem[0]]).sum() == len(mem), "cluster %d is not a whole flat cluster" % c


def check_matches_sklearn_hdbscan(t):
    from sklearn.cluster import HDBSCAN
    for seed, ms, mcs in [(0, 10, 20), (1, 5, 15), (2, 3, 8)]:
        X = _blobs(seed, 80, 5, 6, noise=40)
        n = X.shape[1]
        lo, hi, w = _tree(X, ms)
        mine = t.hdbscan_tail(lo, hi, w, n, mcs)["labels"]
        ref = HDBSCAN(min_cluster_size=mcs, min_samples=ms, algorithm="brute").fit(X.T.astype(np.float64)).labels_
        # tied points (the HDBSCAN page's "ties"): endpoints of tree edges whose weight
        # another tree edge shares exactly; their attachment depends on the order in
        # which equal edges are merged, and either result is correct
        _, inv, cnt = np.unique(w, return_inverse=True, return_counts=True)
        tied = np.zeros(n, bool)
        tied[lo[cnt[inv] > 1]] = True
        tied[hi[cnt[inv] > 1]] = True
        assert tied.sum() < n // 2  # most points still compared
        keep = ~tied
        mine, ref = mine[keep], ref[keep]
        assert ((mine == -1) == (ref == -1)).all(), "noise differs (seed %d)" % seed
        pairs = set(zip(mine[mine >= 0].tolist(), ref[ref >= 0].tolist()))
        assert len(pairs) == len(set(mine[mine >= 0])) == len(set(ref[ref >= 0])), "partition differs (seed %d)" % seed
        assert len(pairs) >= 2


def check_invariants_random(t):
    for seed in range(3):
        X = _blobs(10 + seed, 50, 3, 4, noise=20)
        n = X.shape[1]
        lo, hi, w = _tree(X, 4)
        for mcs in (2, 5, 12, 40):
            r = t.hdbscan_tail(lo, hi, w, n, mcs)
            pts = [e[1] for e in r["entries"] if e[1] < n]
            assert sorted(pts) == list(range(n))
            size = {c: 0 for c in r["birth"]}
            for e in r["entries"]:
                size[e[0]] += e[3]
            for e in r["entries"]:
                if e[1] >= n:
                    assert e[3] == size[e[1]] >= mcs
                    assert e[2] == r["birth"][e[1]] >= r["birth"][e[0]]
            assert size[n] == n
            lab = r["labels"]
            for i, c in enumerate(r["selected"]):
                assert (lab == i).sum() >= mcs


def check_degenerate(t):
    r = t.hdbscan_tail(np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0), 1, 5)
    assert list(r["labels"]) == [-1] and r["entries"] == []
    with pytest.raises(ValueError):
        t.hdbscan_tail(np.zeros(1, np.int64), np.ones(1, np.int64), np.ones(1), 2, 1)
    with pytest.raises(ValueError):  # a cycle is not a tree
        lo, hi, w = _edges([(0, 1, 1.0), (1, 0, 2.0)])
        t.hdbscan_tail(lo, hi, w, 3, 2)


CHECKS = [(f.__name__, f) for f in [
    check_tie_tree_parent_kept, check_tie_tree_boundary_size, check_line_groups_closed_form,
    check_nested_children_win, check_zero_weights, check_tie_order_decides_attachment, check_clusters_are_scipy_single_linkage_cuts,
    check_matches_sklearn_hdbscan, check_invariants_random, check_degenerate]]


@pytest.mark.parametrize("name,fn", CHECKS, ids=[c[0] for c in CHECKS])
def test_pin(name, fn):
    fn(tail_mod)


MUTANTS = {
    # a child of exactly min_cluster_size points not counted as large
    "large_strict": ("la, lb = size[a] >= mcs, size[b] >= mcs", "la, lb = size[a] > mcs, size[b] > mcs"),
    # excess of mass: children win the tie
    "eom_tie_to_children": ("elif st[c] >= sub:", "elif st[c] > sub:"),
    # lambda taken as the distance itself
    "lambda_is_distance": ("return float(\"inf\") if w == 0.0 else 1.0 / w", "return w"),
    # stability without the birth term
    "stability_no_birth": ("st[parent] += 0.0 if lm == b else s * (lm - b)", "st[parent] += s * lm"),
    # the root may be selected
    "root_selectable": ("        if c == n:\n            keep[c] = False", "        if False:\n            keep[c] = False"),
    # children of a split numbered in descending order of their smallest point
    "bfs_child_order": ("key=lambda x: first_min[x])", "key=lambda x: -first_min[x])"),
    # hierarchy merged in (w, hi, lo) order
    "merge_order": ("order = np.lexsort((hi, lo, w))", "order = np.lexsort((lo, hi, w))"),
}


def _mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "hdbscan_tail.py")).read()
    assert src.count(old) == 1, "mutation anchor must be unique: " + name
    p = tmp_path / ("tail_" + name + ".py")
    p.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("tail_mutant_" + name, p)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_tail_mutant(tmp_path, name):
    mod = _mutant(tmp_path, name)
    caught = []
    for cname, fn in CHECKS:
        try:
            fn(mod)
        except Exception:
            caught.append(cname)
            break  # one catching pin is enough
    assert caught, "no pin catches the planted mistake " + name
