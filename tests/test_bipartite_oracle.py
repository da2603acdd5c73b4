"""Pins of the oracle's bipartite kNN-graph assignment (oracle/bipartite.py).

None comes from the oracle itself:
* closed forms: tiny graphs worked out by hand, round by round (two
  components; a score decided by the degree-weighted cluster totals rather than
  the label order; an exact tie that keeps the current label; a decision that
  turns on the 2m of the null model; an isolated right node; the round cap);
* the fixed point, checked in exact rational arithmetic: at convergence every
  spike's label is a best score for its neighbours under the right labels, and
  every right node's label a best score under the left labels.
The second half plants mistakes in a copy of the module; some pin must fail.
"""
import importlib.util
import os
import sys
from fractions import Fraction

import numpy as np
import pytest

from oracle import bipartite as bip_mod

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _run(t, nbr, m, C, init, gamma=1.0, cap=200):
    left, right, rounds = t.assign(np.array(nbr), m, C, np.array(init), gamma, cap)
    return left.tolist(), right.tolist(), rounds


def check_two_components(t):
    """Spikes 0, 1 list right nodes {0, 1}; spikes 2, 3 list {2, 3}; right labels
    start [0, 0, 1, 1].  Round 1: every spike sees one label twice and takes it;
    every right node sees its two spikes' label.  Round 2 moves nothing."""
    nbr = [[0, 1], [0, 1], [2, 3], [2, 3]]
    assert _run(t, nbr, 4, 2, [0, 0, 1, 1]) == ([0, 0, 1, 1], [0, 0, 1, 1], 2)
    # with one round allowed, round 1's right step has still run
    assert _run(t, nbr, 4, 2, [0, 0, 1, 1], cap=1) == ([0, 0, 1, 1], [0, 0, 1, 1], 1)


def check_degree_weighted_totals(t):
    """nbr [[0,1],[1,2],[1,2]] (degrees 1, 3, 2; 2m = 12), right labels [1, 0, 0].
    Spike 0 sees labels 1 and 0 once each: K(1) = 1 and K(0) = 5 give
    1 - 2/12 > 1 - 10/12, so it takes 1 although 0 is the smaller label.  With
    gamma = 0 the two tie and the smaller label wins; then everything is 0."""
    nbr = [[0, 1], [1, 2], [1, 2]]
    assert _run(t, nbr, 3, 2, [1, 0, 0]) == ([1, 0, 0], [1, 0, 0], 2)
    assert _run(t, nbr, 3, 2, [1, 0, 0], gamma=0.0) == ([0, 0, 0], [0, 0, 0], 2)


def check_tie_keeps_current(t):
    """gamma = 0, nbr [[0,1],[1,2],[1,2]], right labels [1, 1, 0].  Round 1: spike
    0 sees [1, 1] -> 1; spikes 1, 2 tie 1 against 0 and, unlabelled, take 0; right
    node 1 then sees [1, 0, 0] -> 0.  Round 2: spike 0 ties 1 (its label) against
    0 and keeps 1; nothing moves."""
    nbr = [[0, 1], [1, 2], [1, 2]]
    assert _run(t, nbr, 3, 2, [1, 1, 0], gamma=0.0) == ([1, 0, 0], [1, 0, 0], 2)


def check_null_model_2m(t):
    """nbr [[1,2],[1,2],[0,2]], right labels [1, 0, 1], gamma = 1, 2m = 12.
    Round 1 left: spikes 0, 1 score 1 - 4/12 for label 0 against 1 - 8/12 for
    label 1 -> 0; spike 2 sees [1, 1] -> 1.  K_left = (4, 2).  Right node 2 sees
    [0, 0, 1]: 2 - 12/12 = 1 against 1 - 6/12 = 0.5 -> 0 (with m instead of 2m
    the two would tie and it would keep 1).  Round 2 moves nothing."""
    nbr = [[1, 2], [1, 2], [0, 2]]
    assert _run(t, nbr, 3, 2, [1, 0, 1]) == ([0, 0, 1], [1, 0, 0], 2)


def check_isolated_right_node(t):
    """A right node that no spike lists keeps its starting label."""
    nbr = [[0, 1], [0, 1]]
    assert _run(t, nbr, 3, 6, [0, 0, 5]) == ([0, 0], [0, 0, 5], 2)


def _best_exact(labels, k_v, K, m_edges, current):
    cands, counts = np.unique(labels, return_counts=True)
    scores = {int(c): Fraction(int(n)) - Fraction(int(k_v) * int(K[c]), 2 * m_edges) for c, n in zip(cands, counts)}
    top = max(scores.values())
    return {c for c, s in scores.items() if s == top}


def check_fixed_point_exact(t):
    rng = np.random.default_rng(5)
    for trial in range(6):
        n, m, k, C = 60, 15, 4, 5
        nbr = np.array([rng.choice(m, k, replace=False) for _ in range(n)])
        init = rng.integers(0, C, m)
        left, right, rounds = t.assign(nbr, m, C, init, 1.0, 200)
        if rounds == 200:
            continue
        m_edges = n * k
        deg = np.bincount(nbr.reshape(-1), minlength=m)
        K_right = np.zeros(C, np.int64)
        np.add.at(K_right, right, deg)
        for i in range(n):
            best = _best_exact(right[nbr[i]], k, K_right, m_edges, left[i])
            assert left[i] in best
        K_left = k * np.bincount(left, minlength=C)
        for r in range(m):
            inc = np.nonzero((nbr == r).any(1))[0]
            if len(inc):
                assert right[r] in _best_exact(left[inc], deg[r], K_left, m_edges, right[r])


CHECKS = [(f.__name__, f) for f in [check_two_components, check_degree_weighted_totals, check_tie_keeps_current,
                                    check_null_model_2m, check_isolated_right_node, check_fixed_point_exact]]


@pytest.mark.parametrize("name,fn", CHECKS, ids=[c[0] for c in CHECKS])
def test_pin(name, fn):
    fn(bip_mod)


MUTANTS = {
    "null_model_m": ("(2.0 * float(m_edges))", "(1.0 * float(m_edges))"),
    "ties_smallest": ("return current if current in best else min(best)", "return min(best)"),
    "totals_by_count": ("K_right = np.bincount(right, weights=deg_r, minlength=n_clusters)",
                        "K_right = np.bincount(right, minlength=n_clusters)"),
    "gain_sign": ("    return float(n_c) - gamma", "    return float(n_c) + gamma"),
    "no_right_step": ("        right = np.array([choose(", "        _unused = np.array([choose("),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_bipartite_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "bipartite.py")).read()
    assert src.count(old) == 1, "mutation anchor must be unique: " + name
    p = tmp_path / ("bip_" + name + ".py")
    p.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("bip_mutant_" + name, p)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    caught = []
    for cname, fn in CHECKS:
        try:
            fn(mod)
        except Exception:
            caught.append(cname)
            break  # one catching pin is enough
    assert caught, "no pin catches the planted mistake " + name
