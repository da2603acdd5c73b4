"""Cluster edge counts and the merging tree of the oracle.

TEST INFRASTRUCTURE ONLY.  Imported by tests/ and bench.py's baseline leg;
never by the product path.  Plain Python and numpy, float64.

Source: the Kilosort4 clustering page, section "Merges and splits": the tree is
built on the host from the cluster-to-cluster edge counts alone (a matrix of at
most 200 x 200 that the device fills and the host copies back once).  The
page does not give the merging rule; the reading taken here stays in the
section "Assignment in parallel"'s modularity terms:

* counts[a, b] = number of kNN edges (spike i, subset point r) with left label
  a = left[i] and right label b = right[r];
* the cluster graph is undirected: W[a, b] = counts[a, b] + counts[b, a] for
  a != b; M = total edges; K[a] = sum_b counts[a, b] + sum_b counts[b, a] (every
  edge adds one end to its left label and one to its right label);
* greedy agglomeration: repeatedly merge the two live clusters a < b with the
  largest modularity gain dQ = W[a, b] / M - gamma K[a] K[b] / (2 M^2), float64
  in exactly that order; ties go to the smallest (a, b) in lexicographic order;
  the merged cluster keeps the id a, with W[a, .] += W[b, .] and K[a] += K[b];
* all C - 1 merges are made (gains may turn negative), so the result is a full
  binary tree, listed as (a, b, dQ) in merge order; with no edges at all every
  gain is 0.
"""
from __future__ import annotations

import numpy as np


def edge_counts(nbr, left, right, n_clusters):
    """counts [C, C] int64 from the kNN edges and both sides' labels."""
    nbr = np.asarray(nbr, np.int64)
    n, k = nbr.shape
    C = n_clusters
    counts = np.zeros((C, C), np.int64)
    for i in range(n):
        a = int(left[i])
        for r in nbr[i]:
            counts[a, int(right[int(r)])] += 1
    return counts


def gain(w_ab, k_a, k_b, m_total, gamma):
    if m_total == 0:
        return 0.0
    return float(w_ab) / float(m_total) - gamma * float(k_a) * float(k_b) / (2.0 * float(m_total) * float(m_total))


def merge_tree(counts, gamma=1.0):
    """Returns a list of (a, b, dQ) for the C - 1 merges."""
    counts = np.asarray(counts, np.int64)
    C = counts.shape[0]
    M = int(counts.sum())
    W = counts + counts.T
    K = counts.sum(1) + counts.sum(0)
    alive = [True] * C
    merges = []
    for _ in range(C - 1):
        best = None
        for a in range(C):
            if not alive[a]:
                continue
            for b in range(a + 1, C):
                if not alive[b]:
                    continue
                g = gain(W[a, b], K[a], K[b], M, gamma)
                if best is None or g > best[2]:
                    best = (a, b, g)
        a, b, g = best
        merges.append((a, b, g))
        alive[b] = False
        W[a, :] += W[b, :]
        W[:, a] += W[:, b]
        K[a] += K[b]
    return merges
