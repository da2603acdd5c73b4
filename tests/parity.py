"""Parity checks of GPU outputs against the float64 oracle.

Rules (tolerances from the accuracy targets of the method: index sets exact
wherever the distance gap exceeds 1e-4 relative; distances, core distances and
total tree weight within 1e-5 relative):

* distances: within 1e-5 relative of the float64 value.  A relative bound
  cannot hold where D is near 0 for the GEMM form (|x|^2 + |y|^2) - 2 x.y, so
  a distance also passes when its square is within an absolute floor
  eps = 4 u (|x|^2 + |y|^2), u = 2^-24, of the true square (the search page's
  policy of a relative 1e-4 equivalence with an absolute floor, the floor sized to
  a few float32 roundings of the norms).  Only distances near 0 can need the
  floor: if the relative test fails and the floor test passes, then
  2e-5 D^2 < |D_gpu^2 - D^2| <= eps.  Every check counts the entries that
  needed it.
* near ties: ranks whose oracle distance is within 1e-4 relative (or the
  floor) of a neighbouring rank may hold either index; elsewhere indices must
  be equal.
* trees: the GPU tree's edges that the oracle's tree lacks must be near-tie
  swaps (no heavier than (1 + 1e-4) x the heaviest oracle edge on the path
  between their ends); per-edge weights, the sorted weight multiset and the
  total weight within 1e-5 relative.
"""
from __future__ import annotations

import numpy as np

import oracle
from treecheck import PathMax, is_spanning_tree, key_less

U = 2.0 ** -24
REL_D = 1e-5   # distances, core distances, edge weights, total weight
REL_GAP = 1e-4  # near-tie class
FLOOR_UNITS = 4  # floor near D = 0, in units of u (|x|^2 + |y|^2)


def sq_norms(X: np.ndarray) -> np.ndarray:
    X64 = X.astype(np.float64)
    return np.einsum("fi,fi->i", X64, X64)


def floor_sq(na, nb):
    """Absolute floor on a squared distance between points of squared norms na, nb."""
    return FLOOR_UNITS * U * (np.asarray(na, np.float64) + np.asarray(nb, np.float64))


def dist_floor(eps2, a, b):
    """A bound on |D_a - D_b| implied by |D_a^2 - D_b^2| <= eps2."""
    eps2 = np.asarray(eps2, np.float64)
    return eps2 / np.maximum(np.asarray(a) + np.asarray(b), np.sqrt(eps2))


def dist_check(g, t, eps2):
    """GPU distances g against float64 distances t: (ok, floor_used, rel_err).

    ok: within REL_D relative, or |g^2 - t^2| <= eps2 (D near 0 only)."""
    g = np.asarray(g, np.float64)
    t = np.asarray(t, np.float64)
    rel_ok = np.abs(g - t) <= REL_D * t
    flo_ok = np.abs(g * g - t * t) <= eps2
    rel = np.where(t > 0, np.abs(g - t) / np.where(t > 0, t, 1.0), np.where(g == t, 0.0, np.inf))
    return rel_ok | flo_ok, (~rel_ok) & flo_ok, rel


def true_sqdist(X, rows, Y, idx):
    """float64 D^2 between X[:, rows[r]] and Y[:, idx[r, t]] by direct differences."""
    Xr = X[:, rows].astype(np.float64)  # [d, r]
    out = np.empty(idx.shape, np.float64)
    for t in range(idx.shape[1]):
        Yt = Y[:, idx[:, t]].astype(np.float64)
        out[:, t] = ((Xr - Yt) ** 2).sum(axis=0)
    return out


def gemm_floor_sq(d, na, nb):
    """Rounding bound of the GEMM-form D2 in float32: the norms and the dot
    product are each d / 4 MFMA steps of 4 products, plus two final roundings."""
    return (d + 4) * U * (np.asarray(na, np.float64) + np.asarray(nb, np.float64))


def check_knn(X, Y, k, gi, gd, rows=None, report=None, rescored=False, gemm_lists=False, nthreads=0):
    """gi, gd: GPU [n, k] (indices into Y, float32 distances) for all rows of X
    (or for ``rows`` only, in that order).  ``rescored``: the distances were
    recomputed by direct differences (ekh_knn), so they must meet the 1e-5
    relative bound with no floor, and each row must ascend in them.
    ``gemm_lists``: the distances are the GEMM-form values that
    ekh_core_distances hands to ekh_mst_boruvka (not a reported distance); they
    are checked against that form's rounding bound instead of 1e-5 relative.
    Indices follow the near-tie rule either way."""
    d, n = X.shape
    m = Y.shape[1]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    gi = np.asarray(gi)[: len(rows)] if gi.shape[0] == len(rows) else np.asarray(gi)[rows]
    gd = np.asarray(gd)[: len(rows)] if gd.shape[0] == len(rows) else np.asarray(gd)[rows]
    assert gi.shape == (len(rows), k)
    kk = min(k + 1, m)
    oi, od2 = oracle.knn(np.ascontiguousarray(X[:, rows]), Y, kk, nthreads=nthreads)
    nx = sq_norms(X)[rows]
    ny = sq_norms(Y)
    # indices valid and distinct per row
    assert gi.min() >= 0 and gi.max() < m, "index out of range"
    srt = np.sort(gi, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]), "repeated index in a row"
    t2 = true_sqdist(X, rows, Y, gi)
    eps_g = floor_sq(nx[:, None], ny[gi])
    eps_o = floor_sq(nx[:, None], ny[oi[:, :k]])
    eps = np.maximum(eps_g, eps_o)
    o2 = od2[:, :k]
    # rank-wise: the GPU's neighbour at rank r is as near as the oracle's rank r
    bad = np.abs(t2 - o2) > 2 * REL_GAP * o2 + eps
    assert not bad.any(), "rank distance mismatch at %d entries, e.g. row %d" % (bad.sum(), rows[np.argwhere(bad)[0][0]])
    # exact indices wherever the oracle's rank is isolated by more than the near-tie class
    tol = 2 * REL_GAP * od2 + floor_sq(nx[:, None], ny[oi])
    R = len(rows)
    gap_prev = np.full((R, k), np.inf)
    gap_prev[:, 1:] = od2[:, 1:k] - od2[:, : k - 1]
    gap_next = np.full((R, k), np.inf)
    nn = min(k, kk - 1)
    gap_next[:, :nn] = od2[:, 1:nn + 1] - od2[:, :nn]
    iso = (gap_prev > tol[:, :k]) & (gap_next > tol[:, :k])
    mism = iso & (gi != oi[:, :k])
    assert not mism.any(), "index mismatch at isolated ranks: %d entries" % mism.sum()
    # reported distances against the float64 distance of the same pair
    dt = np.sqrt(t2)
    ok, used, rel = dist_check(gd, dt, eps_g)
    if gemm_lists:
        ok = np.abs(gd.astype(np.float64) ** 2 - t2) <= gemm_floor_sq(d, nx[:, None], ny[gi])
        used = np.zeros_like(ok)
        assert ok.all(), "list D2 beyond the GEMM form's rounding bound at %d entries" % (~ok).sum()
    assert ok.all(), "distance beyond 1e-5 relative (and the floor near 0) at %d entries" % (~ok).sum()
    if rescored:
        bad = np.abs(gd.astype(np.float64) - dt) > REL_D * dt
        assert not bad.any(), "direct-difference distance beyond 1e-5 relative at %d entries" % bad.sum()
        assert np.all(np.diff(gd, axis=1) >= 0), "rows must ascend in the reported distance"
    if report is not None:
        report.update(rows=int(R), isolated=int(iso.sum()), entries=int(iso.size),
                      max_rel_dist=float(rel[t2 > 0].max(initial=0)), floor_used=int(used.sum()))
    return oi, od2


def check_core(X, ms, gcore, rows=None, report=None, nthreads=0):
    """GPU core distances (all rows, or ``rows``) against the oracle's rank-ms
    distance: 1e-5 relative, the floor near 0 only."""
    d, n = X.shape
    rows = np.arange(n) if rows is None else np.asarray(rows)
    gcore = np.asarray(gcore, np.float64)
    gc = gcore[rows] if gcore.shape[0] == n else gcore
    oi, od2 = oracle.knn(np.ascontiguousarray(X[:, rows]), X, ms, nthreads=nthreads)
    nx = sq_norms(X)
    eps = floor_sq(nx[rows], nx[oi[:, ms - 1]])
    ok, used, rel = dist_check(gc, np.sqrt(od2[:, ms - 1]), eps)
    assert ok.all(), "core distance beyond 1e-5 relative (and the floor near 0) at %d rows" % (~ok).sum()
    if report is not None:
        report.update(max_rel_core=float(rel[od2[:, ms - 1] > 0].max(initial=0)), core_floor_used=int(used.sum()))


def check_core_against(X, gcore, ocore, report=None):
    """GPU core distances against stored float64 oracle core distances (all n).
    The floor uses the bound |b| <= |a| + core_a on the core neighbour b."""
    gcore = np.asarray(gcore, np.float64)
    ocore = np.asarray(ocore, np.float64)
    nx = sq_norms(X)
    eps = floor_sq(nx, (np.sqrt(nx) + ocore) ** 2)
    ok, used, rel = dist_check(gcore, ocore, eps)
    assert ok.all(), "core distance beyond 1e-5 relative (and the floor near 0) at %d points" % (~ok).sum()
    if report is not None:
        report.update(max_rel_core=float(rel[ocore > 0].max(initial=0)), core_floor_used=int(used.sum()))


def check_tree_shape(n, lo, hi, w):
    lo = np.asarray(lo)
    hi = np.asarray(hi)
    w = np.asarray(w)
    assert lo.shape == (n - 1,) and hi.shape == (n - 1,) and w.shape == (n - 1,)
    assert np.all(lo < hi), "edges must have lo < hi"
    assert is_spanning_tree(n, lo, hi), "not a spanning tree"
    # sorted by (w, lo, hi) in the GPU's own float32 weights
    if n > 2:
        w64 = w.astype(np.float64)
        ok = key_less(w64[:-1], lo[:-1], hi[:-1], w64[1:], lo[1:], hi[1:])
        assert ok.all(), "edges not sorted by (w, lo, hi)"


def weight_floor(nx, core, lo, hi):
    """Squared floor of W = max(core_lo, core_hi, D(lo, hi)): the pair's, and
    each core distance's (its neighbour b has |b| <= |a| + core_a)."""
    f_pair = floor_sq(nx[lo], nx[hi])
    f_lo = floor_sq(nx[lo], (np.sqrt(nx[lo]) + core[lo]) ** 2)
    f_hi = floor_sq(nx[hi], (np.sqrt(nx[hi]) + core[hi]) ** 2)
    return np.maximum(f_pair, np.maximum(f_lo, f_hi))


def compare_trees(X, core64, lo, hi, w, olo, ohi, report=None):
    """GPU tree (lo, hi, float32 w; sorted by (w, lo, hi)) against the oracle's
    tree (olo, ohi, any order), both under the float64 weights that the oracle
    computes from its core distances ``core64``.  Returns the mask of GPU edges
    missing from the oracle's tree."""
    d, n = X.shape
    lo = np.asarray(lo).astype(np.int64)
    hi = np.asarray(hi).astype(np.int64)
    w = np.asarray(w).astype(np.float64)
    olo = np.asarray(olo).astype(np.int64)
    ohi = np.asarray(ohi).astype(np.int64)
    check_tree_shape(n, lo, hi, w)
    nx = sq_norms(X)
    # the GPU's edges under float64 weights
    w_t, _ = oracle.pair_weights(X, core64, lo.astype(np.int32), hi.astype(np.int32))
    eps2 = weight_floor(nx, core64, lo, hi)
    ok, used, rel = dist_check(w, w_t, eps2)
    assert ok.all(), "edge weight beyond 1e-5 relative (and the floor near 0) at %d edges" % (~ok).sum()
    # the oracle's edges, in (w, lo, hi) order
    ow, _ = oracle.pair_weights(X, core64, olo.astype(np.int32), ohi.astype(np.int32))
    order = np.lexsort((ohi, olo, ow))
    olo, ohi, ow = olo[order], ohi[order], ow[order]
    # sorted weight multisets (independent of how ties were resolved)
    ws = np.sort(w)
    o_eps2 = weight_floor(nx, core64, olo, ohi)
    eps_sorted = np.maximum(np.sort(eps2), np.sort(o_eps2))
    ok_s, used_s, rel_s = dist_check(ws, ow, eps_sorted)
    assert ok_s.all(), "sorted weights differ beyond 1e-5 relative at %d positions" % (~ok_s).sum()
    # total weight: 1e-5 relative; only edges near 0 (where the floor decides) add their floor
    tot_g, tot_o = float(w.sum()), float(ow.sum())
    near0 = used_s
    tol_total = REL_D * tot_o + float(dist_floor(eps_sorted[near0], ws[near0], ow[near0]).sum())
    assert abs(tot_g - tot_o) <= tol_total, "total weight %.12g vs %.12g (tol %.3g)" % (tot_g, tot_o, tol_total)
    # edges not in the oracle's tree must be near-tie swaps
    key = lambda a, b: a * n + b  # noqa: E731
    extra = ~np.isin(key(lo, hi), key(olo, ohi))
    if extra.any():
        pm = PathMax(n, olo, ohi)
        pmax = ow[pm.query(lo[extra], hi[extra])]
        eps_x = dist_floor(eps2[extra], w_t[extra], pmax)
        bad = w_t[extra] > (1 + REL_GAP) * pmax + eps_x
        assert not bad.any(), "%d GPU edges are not near-tie swaps" % bad.sum()
    if report is not None:
        report.update(n_extra=int(extra.sum()), total_gpu=tot_g, total_oracle=tot_o,
                      rel_total=abs(tot_g - tot_o) / tot_o if tot_o else 0.0,
                      max_rel_w=float(rel[w_t > 0].max(initial=0)), w_floor_used=int(used.sum()),
                      max_rel_sorted_w=float(rel_s[ow > 0].max(initial=0)))
    return extra


def check_mst(X, ms, lo, hi, w, oracle_tree=None, core64=None, report=None):
    """Full comparison with the oracle's tree (small n)."""
    if core64 is None:
        core64 = oracle.core_distances(X, ms)
    if oracle_tree is None:
        oracle_tree = oracle.mst_prim(X, core64)
    olo, ohi, _ = oracle_tree
    return compare_trees(X, core64, lo, hi, w, olo, ohi, report=report)
