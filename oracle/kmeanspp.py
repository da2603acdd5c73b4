"""Greedy k-means++ seeding of the oracle.

TEST INFRASTRUCTURE ONLY.  Imported by tests/ and bench.py's baseline leg;
never by the product path.  Plain Python and numpy.

Source: the Kilosort4 clustering page, section "The measurement that changed
the design: serial chains inside a thread".  Seeds are chosen one after
another; for each seed after the first, 2 + ln k candidates are sampled with
weights proportional to their squared distance to the closest seed chosen so
far, and the candidate giving the lowest potential wins.  The random numbers
are generated on the host and uploaded in one go.  The page states the method, not its arithmetic;
the readings taken here:

* k seeds over the n points (columns) of a feature-major section X [d, n];
  L = 2 + floor(ln k) candidates per seed after the first (7 for the page's
  k = 200, its "seven candidates");
* squared distances in float32, summed feature by feature in feature order from
  0, each subtraction, product and sum rounded to float32 (nothing fused);
* the weights are exact integers: with D1 the squared distances to the first
  seed and 2^(e-1) <= max D1 < 2^e, S = 40 - e (S = 0 when max D1 = 0); a
  squared distance D becomes floor(D * 2^S), exact in float64 because the
  scaling is a power of two; weights stay below 2^40, so all their sums are
  exact in 64 bits whatever the order of summation;
* uniforms are integers u in [0, 2^53), used in order: one for the first seed,
  then L per later seed;
* the first seed is point floor(u n / 2^53) (uniform); a candidate is the first
  point whose inclusive prefix sum of weights exceeds floor(u T / 2^53), T the
  total weight (point 0 when T = 0);
* a candidate's potential is the total weight if it were added:
  sum_x min(w(x), floor(D(x, cand) * 2^S)); the smallest potential wins, ties
  going to the candidate drawn first; then w(x) = min(w(x), floor(D(x, seed) * 2^S)).
"""
from __future__ import annotations

import math

import numpy as np

WEIGHT_BITS = 40
UNIFORM_BITS = 53


def n_candidates(k):
    """Candidates per seed after the first: 2 + floor(ln k)."""
    return 2 + int(math.floor(math.log(k))) if k > 1 else 0


def n_uniforms(k):
    return 1 + (k - 1) * n_candidates(k)


def sqdist_f32(X, c):
    """float32 squared distance of every column of X [d, n] to column c, one
    feature at a time, each operation rounded to float32."""
    X = np.asarray(X, np.float32)
    s = np.zeros(X.shape[1], np.float32)
    for f in range(X.shape[0]):
        v = X[f] - X[f, c]
        s = s + v * v
    return s


def scale_exponent(max_d2):
    """S with max_d2 * 2^S < 2^40 <= 2 max_d2 * 2^S (0 when max_d2 = 0)."""
    if max_d2 == 0.0:
        return 0
    _, e = math.frexp(float(max_d2))  # max_d2 = m 2^e with 0.5 <= m < 1
    return WEIGHT_BITS - e


def weights(d2, S):
    """floor(d2 * 2^S) for each entry, as Python ints."""
    return [int(math.floor(float(v) * (2.0 ** S))) for v in d2]


def first_point(u, n):
    return (int(u) * n) >> UNIFORM_BITS


def draw(w, u):
    """The first index whose inclusive prefix sum of w exceeds floor(u T / 2^53)."""
    total = sum(w)
    t = (int(u) * total) >> UNIFORM_BITS
    acc = 0
    for x, v in enumerate(w):
        acc += v
        if acc > t:
            return x
    return 0


def potential(w, wc):
    return sum(min(a, b) for a, b in zip(w, wc))


def seed(X, k, uniforms):
    """k seed indices (list of int) and the final total weight (int)."""
    X = np.asarray(X, np.float32)
    n = X.shape[1]
    L = n_candidates(k)
    u = [int(v) for v in uniforms]
    assert k >= 1 and n >= 1 and len(u) >= n_uniforms(k)
    first = first_point(u[0], n)
    d1 = sqdist_f32(X, first)
    S = scale_exponent(d1.max())
    w = weights(d1, S)
    seeds = [first]
    pos = 1
    for _ in range(1, k):
        best = None
        for j in range(L):
            cand = draw(w, u[pos + j])
            wc = weights(sqdist_f32(X, cand), S)
            phi = potential(w, wc)
            if best is None or phi < best[0]:
                best = (phi, cand, wc)
        pos += L
        seeds.append(best[1])
        w = [min(a, b) for a, b in zip(w, best[2])]
    return seeds, sum(w)
