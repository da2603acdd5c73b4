"""HDBSCAN tail of the oracle: tree -> hierarchy -> condensed tree -> excess of mass -> labels.

TEST INFRASTRUCTURE ONLY.  Imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg; never by the product path.  Plain Python and
numpy, float64, no blocking or fusion, so that it can be checked against the
definition by eye.

The HDBSCAN page ("The algorithm on the device", last item) places these three
steps on the host and calls them linear, but does not spell them out.  This
module takes the standard definitions of HDBSCAN* (single-linkage hierarchy of
the mutual-reachability tree, condensed by a minimum cluster size, clusters
chosen by excess of mass, i.e. by stability) and fixes every convention the
pages leave open, so that a second implementation can be compared entry for
entry:

* hierarchy: the tree's edges are merged in ascending (w, lo, hi) order (the
  same total order that makes the tree unique), one union per edge;
* lambda = 1 / w, with lambda = +inf for w = 0;
* condensing, walking the hierarchy from the top inside a cluster c: at a merge
  node of distance w with children a and b, a child with at least
  min_cluster_size points is "large".  Both large: c ends and two new clusters
  are born at lambda = 1/w.  One large: the points of the other child leave c at
  lambda, c continues in the large child.  Neither large: all points of both
  children leave c at lambda and c ends;
* cluster ids: the root is n; the others are numbered n + 1, n + 2, ... in
  breadth-first order of the cluster tree, the two children of a split in
  ascending order of their smallest point index;
* condensed-tree entries (parent, child, lambda, size), child a point index
  (size 1) or a cluster id (size = its point count), listed in ascending
  (parent, child) order;
* stability(c) = sum over c's entries, in that order, of size * (lambda -
  birth(c)), a term being 0 when lambda == birth(c) (this also covers
  inf - inf for clusters born at w = 0);
* excess of mass, children before parents (descending id): a non-root cluster
  is kept if its stability is >= the summed best values of its child clusters
  (children summed in ascending id order), and its best value is then its
  stability; otherwise its best value is that sum.  The root is never
  selected.  The selection is the kept clusters with no kept ancestor;
* labels: the selected clusters in ascending id get labels 0, 1, ...; a point
  gets the label of the selected cluster it belongs to (at any depth below it),
  else -1 (noise).

min_cluster_size must be >= 2; n = 1 gives one noise point and no entries.
"""
from __future__ import annotations

import numpy as np


def lam(w):
    """lambda = 1/w, +inf at w = 0 (float64)."""
    w = float(w)
    return float("inf") if w == 0.0 else 1.0 / w


def single_linkage(lo, hi, w, n):
    """Merge the n - 1 tree edges in (w, lo, hi) order.  Returns, for the
    internal nodes n .. 2n - 2 (in merge order), arrays left, right, dist,
    size, and minpt (smallest point index below the node)."""
    lo = np.asarray(lo, np.int64)
    hi = np.asarray(hi, np.int64)
    w = np.asarray(w, np.float64)
    assert lo.shape == hi.shape == w.shape == (n - 1,)
    order = np.lexsort((hi, lo, w))
    uf = list(range(2 * n - 1))  # union-find over node ids; a root's entry is itself

    def find(x):
        r = x
        while uf[r] != r:
            r = uf[r]
        while uf[x] != r:
            uf[x], x = r, uf[x]
        return r

    size = [1] * n + [0] * (n - 1)
    minpt = list(range(n)) + [0] * (n - 1)
    left = [0] * (n - 1)
    right = [0] * (n - 1)
    dist = [0.0] * (n - 1)
    for k, e in enumerate(order):
        a, b = find(int(lo[e])), find(int(hi[e]))
        if a == b:
            raise ValueError("edges do not form a spanning tree (cycle at edge %d)" % e)
        node = n + k
        left[k], right[k], dist[k] = a, b, float(w[e])
        size[node] = size[a] + size[b]
        minpt[node] = min(minpt[a], minpt[b])
        uf[a] = node
        uf[b] = node
    return left, right, dist, size, minpt


def _leaves(node, n, left, right):
    out = []
    stack = [node]
    while stack:
        x = stack.pop()
        if x < n:
            out.append(x)
        else:
            stack.append(left[x - n])
            stack.append(right[x - n])
    return out


def condense(lo, hi, w, n, min_cluster_size):
    """Condensed tree.  Returns (entries, birth) where entries is a list of
    (parent, child, lambda, size) in ascending (parent, child) order and birth
    maps cluster id -> lambda at birth."""
    mcs = int(min_cluster_size)
    if mcs < 2:
        raise ValueError("min_cluster_size must be >= 2")
    if n <= 1:
        return [], {n: 0.0}
    left, right, dist, size, minpt = single_linkage(lo, hi, w, n)
    top = 2 * n - 2
    # raw entries with provisional cluster names, then breadth-first renaming
    raw = []
    kids = {0: []}  # provisional cluster -> provisional child clusters (with their first node)
    birth_p = {0: 0.0}
    first_min = {0: minpt[top]}
    work = [(top, 0)]
    nxt = 1
    while work:
        node, c = work.pop()
        while True:
            k = node - n
            a, b = left[k], right[k]
            lm = lam(dist[k])
            la, lb = size[a] >= mcs, size[b] >= mcs
            if la and lb:
                for ch in (a, b):
                    pc = nxt
                    nxt += 1
                    kids[c].append(pc)
                    kids[pc] = []
                    birth_p[pc] = lm
                    first_min[pc] = minpt[ch]
                    raw.append((c, ("c", pc), lm, size[ch]))
                    work.append((ch, pc))
                break
            if la or lb:
                big, small = (a, b) if la else (b, a)
                for p in _leaves(small, n, left, right):
                    raw.append((c, ("p", p), lm, 1))
                node = big
                continue
            for ch in (a, b):
                for p in _leaves(ch, n, left, right):
                    raw.append((c, ("p", p), lm, 1))
            break
    # breadth-first ids: root n, children of each split by ascending smallest point
    ident = {0: n}
    queue = [0]
    nid = n + 1
    qi = 0
    while qi < len(queue):
        c = queue[qi]
        qi += 1
        for pc in sorted(kids[c], key=lambda x: first_min[x]):
            ident[pc] = nid
            nid += 1
            queue.append(pc)
    entries = []
    for (c, (kind, x), lm, s) in raw:
        child = x if kind == "p" else ident[x]
        entries.append((ident[c], child, lm, s))
    entries.sort(key=lambda e: (e[0], e[1]))
    birth = {ident[c]: b for c, b in birth_p.items()}
    return entries, birth


def stabilities(entries, birth):
    """stability per cluster id, summed over its entries in list order."""
    st = {c: 0.0 for c in birth}
    for parent, child, lm, s in entries:
        b = birth[parent]
        st[parent] += 0.0 if lm == b else s * (lm - b)
    return st


def select_eom(entries, birth, n):
    """Excess-of-mass selection: returns the sorted list of selected cluster ids."""
    st = stabilities(entries, birth)
    children = {c: [] for c in birth}
    for parent, child, lm, s in entries:
        if child >= n:
            children[parent].append(child)
    best = {}
    keep = {}
    for c in sorted(birth, reverse=True):
        sub = 0.0
        for ch in sorted(children[c]):
            sub += best[ch]
        if c == n:
            keep[c] = False
            best[c] = sub
        elif st[c] >= sub:
            keep[c] = True
            best[c] = st[c]
        else:
            keep[c] = False
            best[c] = sub
    # a kept cluster with a kept ancestor is dropped
    selected = []
    stack = [(n, False)]
    while stack:
        c, covered = stack.pop()
        if keep[c] and not covered:
            selected.append(c)
        for ch in children[c]:
            stack.append((ch, covered or keep[c]))
    return sorted(selected)


def labels(entries, birth, n, selected):
    """Label per point: index of its selected cluster in ascending id order, else -1."""
    lab_of = {c: i for i, c in enumerate(sorted(selected))}
    parent_of = {}
    for parent, child, lm, s in entries:
        parent_of[child] = parent
    out = np.full(n, -1, np.int64)
    for p in range(n):
        c = parent_of.get(p)
        while c is not None:
            if c in lab_of:
                out[p] = lab_of[c]
            c = parent_of.get(c)
    return out


def hdbscan_tail(lo, hi, w, n, min_cluster_size):
    """Everything at once: dict with entries, birth, stability, selected, labels."""
    entries, birth = condense(lo, hi, w, n, min_cluster_size)
    sel = select_eom(entries, birth, n)
    lab = labels(entries, birth, n, sel)
    return {"entries": entries, "birth": birth, "stability": stabilities(entries, birth), "selected": sel,
            "labels": lab}
