"""Seeded synthetic point sets for the exact kNN / HDBSCAN hot path.

This module only draws numbers: it holds none of the arithmetic of the method
(no distances, no neighbour lists, no trees), so both the HIP path and the CPU
oracle may take their inputs from it.  Every set is returned feature-major,
``[d, n]`` C-contiguous float32, which is how the clustering page ("k-nearest
neighbours are a matrix product") stores a section embedding.

Workloads (shapes and distributions follow the spike-sorting data the pages
measure on; the recordings themselves are not public, so these stand in):

* ``tiny``      2,000 x 60, mixture of 8 isotropic Gaussians.
* ``ks4_section`` 50,000 x 102, mixture of 40 Gaussians, subset = every 10th point.
* ``wide_section`` 200,000 x 200, 200 Gaussians + 5 % uniform outliers, subset every 10th.
* ``ks4_seeding`` 1,416 x 102, mixture of 40 Gaussians, 200 k-means++ seeds
  (the page's seeding section), with 1 + 199 * 8 uniforms
  (the seeding uses the first 1 + 199 * 7).
* ``clips``     100,000 x 61 biphasic spike clips from 20 templates (HDBSCAN page).
* ``clips_large`` 500,000 x 61 clips from 60 templates + 3 % pure-noise clips.

Draw order inside a generator: parameters, labels, then per-point values.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "WORKLOADS", "make", "gaussian_mixture", "spike_clips", "every_kth",
    "integer_grid", "collinear", "duplicates", "random_uniform",
]


def _to_feature_major(points_nd: np.ndarray) -> np.ndarray:
    """[n, d] float64 -> [d, n] contiguous float32."""
    return np.ascontiguousarray(points_nd.astype(np.float32).T)


def gaussian_mixture(n: int, d: int, n_clusters: int, seed: int = 0, *,
                     means: str = "normal4", sigma: str = "u0.5-1.5",
                     outlier_frac: float = 0.0, outlier_half_width: float = 12.0) -> np.ndarray:
    """Mixture of isotropic Gaussians, feature-major float32 ``[d, n]``.

    means: ``"uniform5"`` -> U[-5, 5]^d ; ``"normal4"`` -> N(0, 4^2)^d.
    sigma: ``"one"`` -> 1 for every cluster ; ``"u0.5-1.5"`` -> U[0.5, 1.5] per cluster.
    A fraction ``outlier_frac`` of the n points (at random positions) is replaced
    by uniform outliers U[-w, w]^d.
    """
    rng = np.random.default_rng(seed)
    if means == "uniform5":
        mu = rng.uniform(-5.0, 5.0, size=(n_clusters, d))
    elif means == "normal4":
        mu = rng.normal(0.0, 4.0, size=(n_clusters, d))
    else:
        raise ValueError(means)
    if sigma == "one":
        sig = np.ones(n_clusters)
    elif sigma == "u0.5-1.5":
        sig = rng.uniform(0.5, 1.5, size=n_clusters)
    else:
        raise ValueError(sigma)
    labels = rng.integers(0, n_clusters, size=n)
    n_out = int(round(outlier_frac * n))
    out_pos = rng.choice(n, size=n_out, replace=False) if n_out else np.zeros(0, np.int64)
    pts = mu[labels] + sig[labels, None] * rng.standard_normal((n, d))
    if n_out:
        pts[out_pos] = rng.uniform(-outlier_half_width, outlier_half_width, size=(n_out, d))
    return _to_feature_major(pts)


def spike_clips(n: int, n_templates: int, seed: int = 0, *, samples: int = 61, peak: int = 20,
                noise_sd: float = 0.1, noise_frac: float = 0.0) -> np.ndarray:
    """Biphasic spike clips, feature-major float32 ``[samples, n]``.

    Template j: T_j(t) = -exp(-(t - peak)^2 / (2 s_j^2)) * cos(2 pi f_j (t - peak)),
    s_j ~ U[2, 4], f_j ~ U[0.08, 0.15]; so T_j(peak) = -1 (a negative peak at
    sample 20 followed by a positive lobe).  A clip is a * T_j + N(0, noise_sd^2)
    with a ~ U[0.5, 2] and j uniform; a fraction ``noise_frac`` of the clips (at
    random positions) is pure noise.
    """
    rng = np.random.default_rng(seed)
    s = rng.uniform(2.0, 4.0, size=n_templates)
    f = rng.uniform(0.08, 0.15, size=n_templates)
    t = np.arange(samples, dtype=np.float64) - peak
    templates = -np.exp(-(t[None, :] ** 2) / (2.0 * s[:, None] ** 2)) * np.cos(2.0 * np.pi * f[:, None] * t[None, :])
    labels = rng.integers(0, n_templates, size=n)
    amp = rng.uniform(0.5, 2.0, size=n)
    n_noise = int(round(noise_frac * n))
    noise_pos = rng.choice(n, size=n_noise, replace=False) if n_noise else np.zeros(0, np.int64)
    pts = amp[:, None] * templates[labels]
    if n_noise:
        pts[noise_pos] = 0.0
    pts += rng.normal(0.0, noise_sd, size=(n, samples))
    return _to_feature_major(pts)


def every_kth(X: np.ndarray, k: int) -> np.ndarray:
    """Columns 0, k, 2k, ... of a feature-major set, gathered contiguous."""
    return np.ascontiguousarray(X[:, ::k])


def random_uniform(n: int, d: int, seed: int = 0, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return _to_feature_major(rng.uniform(lo, hi, size=(n, d)))


def integer_grid(n: int, d: int, seed: int = 0, half_range: int = 8) -> np.ndarray:
    """Integer coordinates in [-half_range, half_range]: small enough that every
    squared distance, norm and dot product is exact in float32, so ties are exact."""
    rng = np.random.default_rng(seed)
    return _to_feature_major(rng.integers(-half_range, half_range + 1, size=(n, d)).astype(np.float64))


def collinear(n: int, d: int, spacing: float = 1.0, axis: int = 0) -> np.ndarray:
    """Points i * spacing along one axis (all other coordinates 0)."""
    pts = np.zeros((n, d))
    pts[:, axis] = spacing * np.arange(n, dtype=np.float64)
    return _to_feature_major(pts)


def duplicates(n_copies: int, d: int, seed: int = 0, n_other: int = 0) -> np.ndarray:
    """``n_copies`` copies of one random point, then ``n_other`` random points."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal(d)
    other = rng.standard_normal((n_other, d)) * 3.0
    return _to_feature_major(np.vstack([np.repeat(base[None, :], n_copies, axis=0), other]))


# name -> (description, factory returning a dict of arrays and parameters)
def random_labels(m: int, n_clusters: int, seed: int = 0) -> np.ndarray:
    """Starting labels for the right nodes of the bipartite assignment: uniform
    in [0, n_clusters), int32 (the page's pipeline seeds them; here they are
    drawn)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, n_clusters, m).astype(np.int32)


def random_neighbour_lists(n: int, m: int, k: int, seed: int = 0) -> np.ndarray:
    """n rows of k distinct indices in [0, m), int32 [n, k]: a kNN-shaped graph
    without the geometry."""
    rng = np.random.default_rng(seed)
    keys = rng.random((n, m))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)


def uniforms53(count: int, seed: int = 0) -> np.ndarray:
    """Uniform integers in [0, 2^53), uint64 [count]: the host-made uniforms
    that the k-means++ seeding consumes."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 53, size=count, dtype=np.uint64)


def _tiny(seed=0):
    X = gaussian_mixture(2000, 60, 8, seed, means="uniform5", sigma="one")
    return {"X": X, "Y": X, "k": 10, "min_samples": 10, "self": True}


def _ks4_section(seed=0):
    X = gaussian_mixture(50_000, 102, 40, seed)
    return {"X": X, "Y": every_kth(X, 10), "k": 10, "self": False}


def _wide_section(seed=0):
    X = gaussian_mixture(200_000, 200, 200, seed, outlier_frac=0.05)
    return {"X": X, "Y": every_kth(X, 10), "k": 10, "self": False, "max_chunk_bytes": 256_000_000}


def _ks4_seeding(seed=0):
    X = gaussian_mixture(1416, 102, 40, seed)
    k = 200
    # enough uniforms for up to 8 candidates per seed (the seeding uses 7)
    return {"X": X, "k": k, "uniforms": uniforms53(1 + (k - 1) * 8, seed + 1)}


def _clips(seed=0):
    X = spike_clips(100_000, 20, seed)
    return {"X": X, "Y": X, "k": 11, "min_samples": 10, "self": True}


def _clips_large(seed=0):
    X = spike_clips(500_000, 60, seed, noise_frac=0.03)
    return {"X": X, "Y": X, "k": 11, "min_samples": 10, "self": True}


WORKLOADS = {
    "tiny_2000x60": _tiny,
    "ks4_section_50000x102": _ks4_section,
    "wide_section_200000x200": _wide_section,
    "ks4_seeding_1416x102": _ks4_seeding,
    "clips_100000x61": _clips,
    "clips_500000x61": _clips_large,
}


def make(name: str, seed: int = 0) -> dict:
    """Build one named workload (see module docstring)."""
    return WORKLOADS[name](seed)
