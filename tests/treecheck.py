"""Checks on spanning trees, shared by the oracle pins and the GPU parity tests.

Pure numpy, no arithmetic of the method beyond what is needed to check a tree:
union-find spanning test, and the maximum edge on the tree path between two
vertices (via the Kruskal reconstruction tree: the path maximum of (a, b) is
the edge at the lowest common ancestor of a and b).
"""
from __future__ import annotations

import numpy as np


def _find(p, x):
    root = x
    while p[root] != root:
        root = p[root]
    while p[x] != root:
        p[x], x = root, p[x]
    return root


def is_spanning_tree(n: int, lo, hi) -> bool:
    lo = np.asarray(lo)
    hi = np.asarray(hi)
    if lo.shape[0] != max(n - 1, 0) or hi.shape[0] != lo.shape[0]:
        return False
    if n <= 1:
        return True
    if lo.min() < 0 or hi.max() >= n or np.any(lo == hi):
        return False
    p = list(range(n))
    for a, b in zip(lo.tolist(), hi.tolist()):
        ra, rb = _find(p, a), _find(p, b)
        if ra == rb:
            return False
        p[ra] = rb
    return True


class PathMax:
    """Maximum-key edge on tree paths.

    Built from a tree whose edges are given in ascending key order; ``query``
    returns, for each pair (a, b), the position (in that order) of the largest
    edge on the path from a to b.
    """

    def __init__(self, n: int, lo, hi):
        lo = np.asarray(lo, np.int64)
        hi = np.asarray(hi, np.int64)
        ne = lo.shape[0]
        assert ne == n - 1
        self.n = n
        size = 2 * n - 1
        parent = np.arange(size, dtype=np.int64)
        uf = list(range(n))
        top = list(range(n))  # current reconstruction-tree node of each union-find root
        for e in range(ne):
            ra, rb = _find(uf, int(lo[e])), _find(uf, int(hi[e]))
            assert ra != rb, "not a tree"
            node = n + e
            parent[top[ra]] = node
            parent[top[rb]] = node
            uf[ra] = rb
            top[rb] = node
        root = size - 1
        depth = np.zeros(size, np.int64)
        # parents always have larger ids, so one sweep from the root down fills depths
        for v in range(size - 2, -1, -1):
            depth[v] = depth[parent[v]] + 1
        depth[root] = 0
        levels = max(1, int(np.ceil(np.log2(max(size, 2)))) + 1)
        up = [parent]
        for _ in range(1, levels):
            up.append(up[-1][up[-1]])
        self.up = up
        self.depth = depth

    def query(self, a, b) -> np.ndarray:
        a = np.asarray(a, np.int64).copy()
        b = np.asarray(b, np.int64).copy()
        swap = self.depth[a] < self.depth[b]
        a[swap], b[swap] = b[swap], a[swap]
        diff = self.depth[a] - self.depth[b]
        for k, upk in enumerate(self.up):
            sel = (diff >> k) & 1 == 1
            a[sel] = upk[a[sel]]
        for upk in reversed(self.up):
            sel = upk[a] != upk[b]
            a[sel] = upk[a[sel]]
            b[sel] = upk[b[sel]]
        lca = np.where(a == b, a, self.up[0][a])
        return lca - self.n  # edge position in ascending key order


def sort_edges(lo, hi, w):
    lo = np.asarray(lo)
    hi = np.asarray(hi)
    w = np.asarray(w)
    order = np.lexsort((hi, lo, w))
    return lo[order], hi[order], w[order]


def key_less(w1, lo1, hi1, w2, lo2, hi2):
    """Vectorised edge order (weight, lower index, higher index)."""
    return (w1 < w2) | ((w1 == w2) & ((lo1 < lo2) | ((lo1 == lo2) & (hi1 < hi2))))
