"""Parity checks of GPU outputs against the float64 oracle.

Rules (tolerances from the accuracy targets of the method: index sets exact
wherever the distance gap exceeds 1e-4 relative; distances, core distances and
total tree weight within 1e-5 relative):

* squared-distance floor: the GEMM form (|x|^2 + |y|^2) - 2 x.y in float32 has
  a rounding error bounded by about (d + 4) u (|x|^2 + |y|^2), u = 2^-24
  (norms: d fmaf steps; dot product: d/4 MFMA steps of 4 products; two final
  roundings).  A relative tolerance cannot hold where D is near 0, so every
  comparison also accepts |D_gpu^2 - D_true^2| <= eps with that bound.
* near ties: ranks whose oracle distance is within 1e-4 relative (or eps) of a
  neighbouring rank may hold either index; elsewhere indices must be equal.
"""
from __future__ import annotations

import numpy as np

import oracle
from treecheck import PathMax, is_spanning_tree, key_less

U = 2.0 ** -24
REL_D = 1e-5   # distances, core distances, total weight
REL_GAP = 1e-4  # near-tie class


def sq_norms(X: np.ndarray) -> np.ndarray:
    X64 = X.astype(np.float64)
    return np.einsum("fi,fi->i", X64, X64)


def floor_sq(d: int, na, nb):
    return (d + 4) * U * (np.asarray(na) + np.asarray(nb))


def dist_floor(eps2, a, b):
    """A bound on |D_a - D_b| implied by |D_a^2 - D_b^2| <= eps2."""
    eps2 = np.asarray(eps2, np.float64)
    return eps2 / np.maximum(np.asarray(a) + np.asarray(b), np.sqrt(eps2))


def true_sqdist(X, rows, Y, idx):
    """float64 D^2 between X[:, rows[r]] and Y[:, idx[r, t]] by direct differences."""
    Xr = X[:, rows].astype(np.float64)  # [d, r]
    out = np.empty(idx.shape, np.float64)
    for t in range(idx.shape[1]):
        Yt = Y[:, idx[:, t]].astype(np.float64)
        out[:, t] = ((Xr - Yt) ** 2).sum(axis=0)
    return out


def check_knn(X, Y, k, gi, gd, rows=None, report=None, rescored=False):
    """gi, gd: GPU [n, k] (indices into Y, float32 distances) for all rows of X
    (or for ``rows`` only, in that order).  ``rescored``: the distances were
    recomputed by direct differences (ekh_knn), so they must meet the 1e-5
    relative bound with no floor, and each row must ascend in them."""
    d, n = X.shape
    m = Y.shape[1]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    gi = np.asarray(gi)[: len(rows)] if gi.shape[0] == len(rows) else np.asarray(gi)[rows]
    gd = np.asarray(gd)[: len(rows)] if gd.shape[0] == len(rows) else np.asarray(gd)[rows]
    assert gi.shape == (len(rows), k)
    kk = min(k + 1, m)
    oi, od2 = oracle.knn(np.ascontiguousarray(X[:, rows]), Y, kk)
    nx = sq_norms(X)[rows]
    ny = sq_norms(Y)
    # indices valid and distinct per row
    assert gi.min() >= 0 and gi.max() < m, "index out of range"
    srt = np.sort(gi, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]), "repeated index in a row"
    t2 = true_sqdist(X, rows, Y, gi)
    eps_g = floor_sq(d, nx[:, None], ny[gi])
    eps_o = floor_sq(d, nx[:, None], ny[oi[:, :k]])
    eps = np.maximum(eps_g, eps_o)
    o2 = od2[:, :k]
    # rank-wise: the GPU's neighbour at rank r is as near as the oracle's rank r
    bad = np.abs(t2 - o2) > 2 * REL_GAP * o2 + eps
    assert not bad.any(), "rank distance mismatch at %d entries, e.g. row %d" % (bad.sum(), rows[np.argwhere(bad)[0][0]])
    # exact indices wherever the oracle's rank is isolated by more than the near-tie class
    tol = 2 * REL_GAP * od2 + floor_sq(d, nx[:, None], ny[oi])
    R = len(rows)
    gap_prev = np.full((R, k), np.inf)
    gap_prev[:, 1:] = od2[:, 1:k] - od2[:, : k - 1]
    gap_next = np.full((R, k), np.inf)
    nn = min(k, kk - 1)
    gap_next[:, :nn] = od2[:, 1:nn + 1] - od2[:, :nn]
    iso = (gap_prev > tol[:, :k]) & (gap_next > tol[:, :k])
    mism = iso & (gi != oi[:, :k])
    assert not mism.any(), "index mismatch at isolated ranks: %d entries" % mism.sum()
    # reported distances
    g2 = gd.astype(np.float64) ** 2
    derr = np.abs(g2 - t2)
    bad = derr > 2 * REL_D * t2 + eps_g
    assert not bad.any(), "distance error beyond tolerance at %d entries" % bad.sum()
    if rescored:
        dt = np.sqrt(t2)
        bad = np.abs(gd.astype(np.float64) - dt) > REL_D * dt
        assert not bad.any(), "direct-difference distance beyond 1e-5 relative at %d entries" % bad.sum()
        assert np.all(np.diff(gd, axis=1) >= 0), "rows must ascend in the reported distance"
    if report is not None:
        rel = np.abs(gd.astype(np.float64) - np.sqrt(t2)) / np.maximum(np.sqrt(t2), 1e-300)
        report.update(isolated=int(iso.sum()), entries=int(iso.size), max_rel_dist=float(rel[t2 > 0].max(initial=0)),
                      floor_used=int(((np.abs(gd - np.sqrt(t2)) > REL_D * np.sqrt(t2)) & ~bad).sum()))
    return oi, od2


def check_core(X, ms, gcore, rows=None, report=None):
    d, n = X.shape
    rows = np.arange(n) if rows is None else np.asarray(rows)
    gcore = np.asarray(gcore, np.float64)
    gc = gcore[rows] if gcore.shape[0] == n else gcore
    oi, od2 = oracle.knn(np.ascontiguousarray(X[:, rows]), X, ms)
    nx = sq_norms(X)
    eps = floor_sq(d, nx[rows], nx[oi[:, ms - 1]])
    o2 = od2[:, ms - 1]
    err = np.abs(gc ** 2 - o2)
    bad = err > 2 * REL_D * o2 + eps
    assert not bad.any(), "core distance mismatch at %d rows" % bad.sum()
    if report is not None:
        report.update(max_rel_core=float((np.abs(gc - np.sqrt(o2)) / np.maximum(np.sqrt(o2), 1e-300))[o2 > 0].max(initial=0)))


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


def check_mst(X, ms, lo, hi, w, oracle_tree=None, core64=None, report=None):
    """Full comparison with the oracle's tree (small n)."""
    d, n = X.shape
    lo = np.asarray(lo).astype(np.int64)
    hi = np.asarray(hi).astype(np.int64)
    w = np.asarray(w).astype(np.float64)
    check_tree_shape(n, lo, hi, w)
    if core64 is None:
        core64 = oracle.core_distances(X, ms)
    if oracle_tree is None:
        oracle_tree = oracle.mst_prim(X, core64)
    olo, ohi, ow = oracle_tree
    # weights of the GPU's edges against their float64 values
    w_t, dist_t = oracle.pair_weights(X, core64, lo.astype(np.int32), hi.astype(np.int32))
    nx = sq_norms(X)
    # W is a core distance or a pair distance: the squared floor of the pair, or of
    # the largest norms for the core neighbours, bounds its float32 error
    eps2 = floor_sq(d, nx[lo], nx[hi]) + floor_sq(d, nx.max(), nx.max())
    eps_w = dist_floor(eps2, w, w_t)
    bad = np.abs(w - w_t) > REL_D * w_t + eps_w
    assert not bad.any(), "edge weight mismatch at %d edges" % bad.sum()
    # total weight
    tot_g, tot_o = float(w_t.sum()), float(ow.sum())
    assert abs(float(w.sum()) - tot_o) <= REL_D * tot_o + eps_w.sum(), "total weight mismatch"
    # edges not in the oracle's tree must be near-tie swaps (cycle property with tolerance)
    okey = set(zip(olo.tolist(), ohi.tolist()))
    extra = np.array([(a, b) not in okey for a, b in zip(lo.tolist(), hi.tolist())])
    if extra.any():
        pm = PathMax(n, olo, ohi)
        pos = pm.query(lo[extra], hi[extra])
        pmax = ow[pos]
        bad = w_t[extra] > (1 + REL_GAP) * pmax + eps_w[extra]
        assert not bad.any(), "%d GPU edges are not near-tie swaps" % bad.sum()
    if report is not None:
        report.update(n_extra=int(extra.sum()), total_gpu=float(w.sum()), total_oracle=tot_o,
                      rel_total=abs(float(w.sum()) - tot_o) / tot_o if tot_o else 0.0,
                      max_rel_w=float((np.abs(w - w_t) / np.maximum(w_t, 1e-300))[w_t > 0].max(initial=0)))
    return extra
