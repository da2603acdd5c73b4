"""Bipartite kNN-graph assignment of the oracle.

TEST INFRASTRUCTURE ONLY.  Imported by tests/ and bench.py's baseline leg;
never by the product path.  Plain Python and numpy, float64.

Source: the Kilosort4 clustering page, section "Assignment in parallel: why
the graph is bipartite".  The spikes form the left side of the graph and a
copy of the subset the right side; each kNN link (spike i, its neighbour r
among the subset) is an edge.  Holding the right labels fixed makes the spikes' choices independent of
one another, so the left side is relabelled in one step, then the right side,
and the two steps alternate.

The page gives the right step's score, n_rc - gamma k_r K_c / 2m, and says that
the left step counts a spike's neighbours' labels and takes the best.  The
readings taken where it is silent:

* m is the number of edges, k_v the degree of node v (k for every spike, the
  number of spikes listing r for a right node), and K_c the total degree of the
  nodes of the OTHER side that carry label c (the side whose labels are being
  counted).  The same score is used in both steps;
* score = n - gamma * k_v * K_c / (2 m), evaluated in float64 in exactly that
  order (n - ((gamma * k_v) * K_c) / (2 m));
* candidates are the labels present among the node's neighbours;
* ties keep the node's current label if it is among the best, else take the
  smallest label;
* spikes start unlabelled (-1); the right nodes start from given labels (the
  page's pipeline seeds them; here they are an input);
* a round is a left step then a right step; the loop stops after a left step
  that moves no spike (the right step would then repeat itself), or after
  max_rounds rounds (the page: a 200-round cap that is never reached);
* a right node with no edges keeps its label.
"""
from __future__ import annotations

import numpy as np


def score(n_c, k_v, K_c, m_edges, gamma):
    """n - gamma k_v K_c / (2 m) in float64, in this order."""
    return float(n_c) - gamma * float(k_v) * float(K_c) / (2.0 * float(m_edges))


def choose(labels, k_v, K, m_edges, gamma, current):
    """Best label among `labels` (the neighbours' labels, with repeats)."""
    cands, counts = np.unique(np.asarray(labels), return_counts=True)
    best, best_s = [], None
    for c, n_c in zip(cands.tolist(), counts.tolist()):
        s = score(n_c, k_v, K[c], m_edges, gamma)
        if best_s is None or s > best_s:
            best, best_s = [c], s
        elif s == best_s:
            best.append(c)
    return current if current in best else min(best)


def assign(nbr, m, n_clusters, init_right, gamma=1.0, max_rounds=200):
    """nbr [n, k] int (right-node indices); returns (left labels [n], right labels
    [m], rounds run)."""
    nbr = np.asarray(nbr, np.int64)
    n, k = nbr.shape
    m_edges = n * k
    deg_r = np.bincount(nbr.reshape(-1), minlength=m)
    # in-edges of every right node: the spikes that list it
    incoming = [[] for _ in range(m)]
    for i in range(n):
        for r in nbr[i]:
            incoming[int(r)].append(i)
    left = np.full(n, -1, np.int64)
    right = np.asarray(init_right, np.int64).copy()
    rounds = 0
    for rnd in range(1, max_rounds + 1):
        rounds = rnd
        K_right = np.bincount(right, weights=deg_r, minlength=n_clusters)  # degrees of right nodes per label
        new_left = np.array([choose(right[nbr[i]], k, K_right, m_edges, gamma, int(left[i])) for i in range(n)],
                            np.int64)
        moved = int((new_left != left).sum())
        left = new_left
        if moved == 0:
            break
        K_left = k * np.bincount(left, minlength=n_clusters)
        right = np.array([choose(left[incoming[r]], deg_r[r], K_left, m_edges, gamma, int(right[r]))
                          if deg_r[r] > 0 else int(right[r]) for r in range(m)], np.int64)
    return left, right, rounds
