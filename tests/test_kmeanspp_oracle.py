"""Pins of the oracle's greedy k-means++ seeding (oracle/kmeanspp.py).

Hand-worked cases in exact binary arithmetic: the candidate count 2 + ln k
(seven at the page's k = 200), float32 rounding and feature order of the
squared distance, the power-of-two weight scale, the prefix-sum draw, a 1-D
seeding worked by hand (the best candidate is not the first drawn), a tie that
goes to the first drawn candidate, and k = 1.  Invariants on random sets: the
returned potential is the floor-scaled distance to the nearest seed summed
over the points, seeds are distinct, well-separated blobs get one seed each,
and draws follow the weights (a frequency test).  Mistakes planted in a copy
of the module must be caught.
"""
import importlib.util
import math
import os
import sys

import numpy as np
import pytest

from exact_knn_hdbscan_amd import datagen
from oracle import kmeanspp as km_mod

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
U = 1 << 53


def fm(points):
    """[n, d] list -> feature-major float32 [d, n]."""
    return np.ascontiguousarray(np.array(points, np.float64).astype(np.float32).T)


def check_candidate_count(t):
    """2 + floor(ln k): ln 200 = 5.30 -> 7 (the page's seven candidates);
    ln 7 = 1.95, ln 8 = 2.08, ln 20 = 3.00, ln 21 = 3.04."""
    got = [t.n_candidates(k) for k in (1, 2, 3, 7, 8, 20, 21, 200)]
    assert got == [0, 2, 3, 3, 4, 4, 5, 7]
    assert t.n_uniforms(200) == 1 + 199 * 7


def check_float32_rounding(t):
    """(1 + 2^-12)^2 = 1 + 2^-11 + 2^-24 is a tie at float32 and rounds to the
    even 1 + 2^-11; features (1, 1, 4096) sum as 1, 2, 2 + 2^24 (exact), while
    (4096, 1, 1) sums as 2^24, then 2^24 + 1 twice, each a tie back to 2^24.
    Features (2^-12, 1 + 2^-12): 2^-24, then the product rounds to 1 + 2^-11
    and 2^-24 + 1 + 2^-11 is a tie back to 1 + 2^-11; a fused multiply-add
    would give the exact 1 + 2^-11 + 2^-23."""
    d2 = t.sqdist_f32(fm([[1 + 2.0 ** -12], [0.0]]), 1)
    assert d2.dtype == np.float32 and d2[0] == np.float32(1 + 2.0 ** -11) and d2[1] == 0
    assert t.sqdist_f32(fm([[1, 1, 4096], [0, 0, 0]]), 1)[0] == 2.0 ** 24 + 2
    assert t.sqdist_f32(fm([[4096, 1, 1], [0, 0, 0]]), 1)[0] == 2.0 ** 24
    assert t.sqdist_f32(fm([[2.0 ** -12, 1 + 2.0 ** -12], [0, 0]]), 1)[0] == 1 + 2.0 ** -11


def check_scale_and_weights(t):
    """max 1 = 0.5 * 2^1 -> S = 39; 0.75 -> 40; 3 = 0.75 * 2^2 -> 38; 2^30 -> 9."""
    assert [t.scale_exponent(v) for v in (1.0, 0.75, 3.0, 2.0 ** 30, 0.0)] == [39, 40, 38, 9, 0]
    assert t.weights(np.array([1.0, 0.5, 0.0, 0.75], np.float32), 39) == [2 ** 39, 2 ** 38, 0, 3 * 2 ** 37]
    assert t.weights(np.array([1 / 3, 2 / 3], np.float32), 2) == [1, 2]   # floor(1.33..), floor(2.66..)


def check_first_point(t):
    assert [t.first_point(0, 7), t.first_point(U // 2, 3), t.first_point(U - 1, 5), t.first_point(U // 2, 2)] \
        == [0, 1, 4, 1]


def check_draw(t):
    """w = (0, 3, 0, 5), T = 8: t = 0 -> 1 (not 0: its prefix 0 does not exceed
    0); t = 3 -> 3; u just under 3/8 -> t = 2 -> 1; t = 7 -> 3; T = 0 -> 0."""
    w = [0, 3, 0, 5]
    assert t.draw(w, 0) == 1
    assert t.draw(w, 3 * U // 8) == 3
    assert t.draw(w, 3 * U // 8 - 1) == 1
    assert t.draw(w, U - 1) == 3
    assert t.draw([0, 0, 0], U // 2) == 0


def check_hand_worked_line(t):
    """Points 0, 1, 3 on a line, k = 2 (L = 2), first = point 0: D2 = (0, 1, 9),
    S = 36, w = (0, 1, 9) 2^36, T = 10 2^36.  u = 2^52 -> t = 5 2^36 -> point 2,
    potential sum min(w, (9, 4, 0) 2^36) = 2^36; u = 0 -> point 1, potential
    sum min(w, (1, 0, 4) 2^36) = 4 2^36.  Point 2 wins in either draw order."""
    X = fm([[0.0], [1.0], [3.0]])
    assert t.seed(X, 2, [0, U // 2, 0]) == ([0, 2], 2 ** 36)
    assert t.seed(X, 2, [0, 0, U // 2]) == ([0, 2], 2 ** 36)


def check_tie_first_drawn(t):
    """Points -1, 0, 1, first = point 1 (u = 2^52): w = (1, 0, 1) 2^39.  u = 0
    draws point 0, u = 2^52 (t = 2^39) draws point 2; both leave 2^39, so the
    first drawn wins."""
    X = fm([[-1.0], [0.0], [1.0]])
    assert t.seed(X, 2, [U // 2, 0, U // 2]) == ([1, 0], 2 ** 39)
    assert t.seed(X, 2, [U // 2, U // 2, 0]) == ([1, 2], 2 ** 39)


def check_single_seed(t):
    """k = 1: the first point only; the potential is sum floor(D2 2^S) with
    D2 = (9, 0, 16, 1) from point 1 of (3, 0, -4, 1) on a line, S = 35."""
    X = fm([[3.0], [0.0], [-4.0], [1.0]])
    assert t.seed(X, 1, [U // 4]) == ([1], 26 * 2 ** 35)


def brute_potential(X, seeds):
    """floor(min over seeds of the float64 squared distance of float32 inputs,
    scaled by 2^S), summed: agrees with the oracle's float32 sums wherever
    those are exact (small integer coordinates)."""
    X64 = np.asarray(X, np.float64)
    d2 = np.min([((X64 - X64[:, [s]]) ** 2).sum(0) for s in seeds], axis=0)
    d1 = ((X64 - X64[:, [seeds[0]]]) ** 2).sum(0)
    _, e = math.frexp(float(d1.max()))
    S = 40 - e
    return int(sum(int(math.floor(v * 2.0 ** S)) for v in d2))


def check_potential_invariant(t):
    """On integer grids every float32 distance is exact, so the returned
    potential must equal the brute-force nearest-seed sum."""
    for seed, (n, d, k) in enumerate([(60, 3, 5), (200, 8, 12), (31, 2, 30)]):
        X = datagen.integer_grid(n, d, seed, half_range=6)
        u = datagen.uniforms53(t.n_uniforms(k), seed)
        seeds, phi = t.seed(X, k, u)
        assert len(seeds) == k
        assert phi == brute_potential(X, seeds)
        n_distinct = len({tuple(c) for c in X.T.tolist()})
        if n_distinct >= k:
            assert len(set(seeds)) == k


def check_separated_blobs(t):
    """Six blobs 1000 apart with unit spread: the chance that a seed lands in an
    already seeded blob is about 1e-6 per draw, so each blob gets one seed."""
    rng = np.random.default_rng(5)
    centres = np.eye(6) * 1000.0
    lab = np.repeat(np.arange(6), 30)
    X = fm(centres[lab] + rng.standard_normal((180, 6)))
    seeds, _ = t.seed(X, 6, datagen.uniforms53(t.n_uniforms(6), 3))
    assert sorted(lab[seeds].tolist()) == list(range(6))


def check_draw_frequencies(t):
    """20,000 draws over weights (5, 0, 1, 10, 4): each count within 5 sigma of
    the binomial mean."""
    w = [5, 0, 1, 10, 4]
    u = datagen.uniforms53(20000, 11)
    counts = np.bincount([t.draw(w, v) for v in u], minlength=5)
    p = np.array(w) / sum(w)
    mean = 20000 * p
    sd = np.sqrt(20000 * p * (1 - p))
    assert counts[1] == 0
    assert np.all(np.abs(counts - mean) <= 5 * sd + 1e-9)


CHECKS = [(f.__name__, f) for f in [
    check_candidate_count, check_float32_rounding, check_scale_and_weights, check_first_point, check_draw,
    check_hand_worked_line, check_tie_first_drawn, check_single_seed, check_potential_invariant,
    check_separated_blobs, check_draw_frequencies]]


@pytest.mark.parametrize("name,fn", CHECKS, ids=[c[0] for c in CHECKS])
def test_pin(name, fn):
    fn(km_mod)


MUTANTS = {
    "candidates_minus_one": ("return 2 + int(math.floor(math.log(k)))", "return 1 + int(math.floor(math.log(k)))"),
    "float64_sum": ("s = s + v * v", "s = (s.astype(np.float64) + v.astype(np.float64) ** 2).astype(np.float32)"),
    "reversed_features": ("for f in range(X.shape[0]):", "for f in reversed(range(X.shape[0])):"),
    "scale_off_by_one": ("return WEIGHT_BITS - e", "return WEIGHT_BITS - e + 1"),
    "first_point_n_minus_1": ("return (int(u) * n) >> UNIFORM_BITS", "return (int(u) * (n - 1)) >> UNIFORM_BITS"),
    "prefix_not_strict": ("if acc > t:", "if acc >= t:"),
    "largest_potential": ("if best is None or phi < best[0]:", "if best is None or phi > best[0]:"),
    "tie_last_drawn": ("if best is None or phi < best[0]:", "if best is None or phi <= best[0]:"),
    "potential_ignores_w": ("return sum(min(a, b) for a, b in zip(w, wc))", "return sum(wc)"),
    "weights_not_kept": ("w = [min(a, b) for a, b in zip(w, best[2])]", "w = best[2]"),
    "weights_round": ("int(math.floor(float(v) * (2.0 ** S)))", "int(round(float(v) * (2.0 ** S)))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_kmeanspp_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(os.path.join(ORACLE_DIR, "kmeanspp.py")).read()
    assert src.count(old) == 1, "mutation anchor must be unique: " + name
    p = tmp_path / ("km_" + name + ".py")
    p.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("km_mutant_" + name, p)
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
