"""Pins of the oracle's cluster edge counts and merging tree (oracle/merge_tree.py).

Hand-worked cases in exact binary fractions: a merge order set by the null
model, a chain merged by connectivity alone (gamma = 0), a tie that goes to the
lexicographically smallest pair, a graph with no edges, and the counts of a
tiny labelled kNN graph.  Mistakes planted in a copy of the module must be
caught.
"""
import importlib.util
import os
import sys

import numpy as np
import pytest

from oracle import merge_tree as mt_mod

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def check_null_model_order(t):
    """counts [[5,3,0],[2,5,0],[0,0,5]]: M = 20, W01 = 5, K = (15, 15, 10).
    dQ01 = 5/20 - 225/800 = -1/32; dQ02 = dQ12 = -150/800 = -3/16, so (0, 1)
    first; then K0 = 30: dQ02 = -300/800 = -3/8."""
    assert t.merge_tree(np.array([[5, 3, 0], [2, 5, 0], [0, 0, 5]])) == [(0, 1, -1 / 32), (0, 2, -3 / 8)]


def check_chain_by_connectivity(t):
    """gamma = 0, a chain 0-1 (1 edge), 1-2 (2), 2-3 (3), M = 6: (2, 3) at 3/6,
    then (1, 2) at 2/6, then (0, 1) at 1/6."""
    c = np.zeros((4, 4), np.int64)
    c[0, 1], c[1, 2], c[2, 3] = 1, 2, 3
    assert t.merge_tree(c, gamma=0.0) == [(2, 3, 3 / 6), (1, 2, 2 / 6), (0, 1, 1 / 6)]


def check_tie_smallest_pair(t):
    """Edges 0-1 and 0-2, M = 2, K = (2, 1, 1): dQ01 = dQ02 = 1/2 - 2/8 = 1/4,
    so (0, 1); then K0 = 3, W02 = 1: 1/2 - 3/8 = 1/8."""
    c = np.zeros((3, 3), np.int64)
    c[0, 1], c[0, 2] = 1, 1
    assert t.merge_tree(c) == [(0, 1, 0.25), (0, 2, 0.125)]


def check_no_edges(t):
    assert t.merge_tree(np.zeros((3, 3), np.int64)) == [(0, 1, 0.0), (0, 2, 0.0)]


def check_edge_counts(t):
    """Spikes 0, 1 (labels 0, 1) list right nodes [0, 1] and [1, 2] (labels 1, 0, 1)."""
    c = t.edge_counts(np.array([[0, 1], [1, 2]]), np.array([0, 1]), np.array([1, 0, 1]), 2)
    assert c.tolist() == [[1, 1], [1, 1]]
    c = t.edge_counts(np.array([[0, 1], [1, 2]]), np.array([1, 1]), np.array([0, 0, 1]), 2)
    assert c.tolist() == [[0, 0], [3, 1]]


CHECKS = [(f.__name__, f) for f in [check_null_model_order, check_chain_by_connectivity, check_tie_smallest_pair,
                                    check_no_edges, check_edge_counts]]


@pytest.mark.parametrize("name,fn", CHECKS, ids=[c[0] for c in CHECKS])
def test_pin(name, fn):
    fn(mt_mod)


MUTANTS = {
    "one_direction": ("W = counts + counts.T", "W = counts.copy()"),
    "degree_one_side": ("K = counts.sum(1) + counts.sum(0)", "K = 2 * counts.sum(1)"),
    "null_model_m2": ("(2.0 * float(m_total) * float(m_total))", "(float(m_total) * float(m_total))"),
    "tie_last_pair": ("if best is None or g > best[2]:", "if best is None or g >= best[2]:"),
    "keep_b": ("        alive[b] = False", "        alive[a] = False"),
    "counts_transposed": ("counts[a, int(right[int(r)])] += 1", "counts[int(right[int(r)]), a] += 1"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_merge_tree_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "merge_tree.py")).read()
    assert src.count(old) == 1, "mutation anchor must be unique: " + name
    p = tmp_path / ("mt_" + name + ".py")
    p.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("mt_mutant_" + name, p)
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
