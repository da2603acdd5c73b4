"""GPU parity of the greedy k-means++ seeding (ekh_kmeanspp) with the oracle.

Every decision is an exact integer comparison on weights computed from the
same float32 bits on both sides, so the bar is exact: identical seed indices
and identical final potential, on both of the library's paths (the
distance-matrix block for small sections, two launches per seed otherwise,
which the flag EKH_KMEANSPP_PER_SEED_LAUNCHES forces).  Cases: the oracle's
hand-worked sets, random
sets over sizes that span one and several point blocks and select passes (with
ragged tails and padded leading dimensions), integer grids full of exact ties,
duplicate points (fewer distinct points than seeds), the Kilosort4 seeding
section at full size (1,416 x 102, 200 seeds), repeatability, the 53-bit mask
of the uniforms, and argument errors.
"""
import numpy as np
import pytest
import torch

import exact_knn_hdbscan_amd as ekh
from exact_knn_hdbscan_amd import binding, datagen
from gpu_util import say
from oracle import kmeanspp as okm

pytestmark = pytest.mark.gpu
U = 1 << 53


def run_gpu(X, k, u, pad=0, per_seed=False):
    d, n = X.shape
    Xt = torch.zeros((d, n + pad), dtype=torch.float32, device="cuda")
    Xt[:, :n] = torch.from_numpy(np.ascontiguousarray(X, np.float32))
    ut = torch.from_numpy(np.asarray(u, np.uint64).astype(np.int64)).cuda()
    seeds, pot = ekh.kmeanspp(Xt[:, :n], k, ut, per_seed_launches=per_seed)
    return seeds.cpu().numpy().tolist(), int(pot.item())


_ORACLE = {}


def oracle_seed(X, k, u):
    """The oracle's seeding, computed once per input (both paths compare to it)."""
    key = (X.shape, k, hash(np.ascontiguousarray(X, np.float32).tobytes()), hash(np.asarray(u, np.uint64).tobytes()))
    if key not in _ORACLE:
        _ORACLE[key] = okm.seed(X, k, u)
    return _ORACLE[key]


def same_as_oracle(X, k, u, pad=0, per_seed=False):
    got = run_gpu(X, k, u, pad, per_seed)
    want = oracle_seed(X, k, u)
    assert got[0] == want[0], "first differing seed at %d" % next(i for i, (a, b) in enumerate(zip(got[0], want[0]))
                                                                   if a != b)
    assert got[1] == want[1]
    return got


def fm(points):
    return np.ascontiguousarray(np.array(points, np.float64).astype(np.float32).T)


@pytest.mark.parametrize("per_seed", [False, True])
def test_hand_worked_sets(per_seed):
    line = fm([[0.0], [1.0], [3.0]])
    assert run_gpu(line, 2, [0, U // 2, 0], per_seed=per_seed) == ([0, 2], 2 ** 36)
    assert run_gpu(line, 2, [0, 0, U // 2], per_seed=per_seed) == ([0, 2], 2 ** 36)
    sym = fm([[-1.0], [0.0], [1.0]])
    assert run_gpu(sym, 2, [U // 2, 0, U // 2], per_seed=per_seed) == ([1, 0], 2 ** 39)
    assert run_gpu(sym, 2, [U // 2, U // 2, 0], per_seed=per_seed) == ([1, 2], 2 ** 39)
    assert run_gpu(fm([[3.0], [0.0], [-4.0], [1.0]]), 1, [U // 4], per_seed=per_seed) == ([1], 26 * 2 ** 35)
    # rounding: features (2^-12, 1 + 2^-12) -> 1 + 2^-11 (not the fused 1 + 2^-11 + 2^-23); S = 39
    X = fm([[2.0 ** -12, 1 + 2.0 ** -12], [0.0, 0.0]])
    assert run_gpu(X, 1, [0], per_seed=per_seed) == ([0], (1 << 39) + (1 << 28))
    assert run_gpu(X, 2, [0, 0, 0], per_seed=per_seed) == ([0, 1], 0)


@pytest.mark.parametrize("per_seed", [False, True])
@pytest.mark.parametrize("n,d,k,pad,seed", [
    (1, 4, 1, 0, 0), (2, 3, 2, 1, 1), (3, 1, 3, 0, 2), (255, 8, 12, 3, 3), (256, 61, 30, 0, 4),
    (257, 102, 50, 5, 5), (1000, 1, 20, 0, 6), (1416, 102, 200, 7, 7), (4097, 16, 40, 0, 8),
    (9000, 5, 25, 11, 9), (700, 200, 100, 0, 10), (4096, 33, 400, 0, 11), (3001, 300, 400, 2, 12)])
def test_random_sets(n, d, k, pad, seed, per_seed):
    X = datagen.gaussian_mixture(n, d, max(1, min(n, 12)), seed)
    u = datagen.uniforms53(okm.n_uniforms(k), seed + 50)
    seeds, pot = same_as_oracle(X, k, u, pad, per_seed)
    say("n %d d %d k %d: potential %d, %d distinct seeds" % (n, d, k, pot, len(set(seeds))))


@pytest.mark.parametrize("per_seed", [False, True])
@pytest.mark.parametrize("n,d,k,seed", [(500, 3, 40, 0), (2000, 2, 64, 1), (300, 4, 300, 2)])
def test_integer_grids_with_ties(n, d, k, seed, per_seed):
    X = datagen.integer_grid(n, d, seed, half_range=3)
    u = datagen.uniforms53(okm.n_uniforms(k), seed + 7)
    same_as_oracle(X, k, u, per_seed=per_seed)


@pytest.mark.parametrize("per_seed", [False, True])
def test_duplicates_fewer_distinct_than_seeds(per_seed):
    X = datagen.duplicates(50, 6, 0, n_other=5)  # 6 distinct points, 20 seeds
    u = datagen.uniforms53(okm.n_uniforms(20), 1)
    seeds, pot = same_as_oracle(X, 20, u, per_seed=per_seed)
    assert pot == 0 and len(set(seeds)) <= 7
    X = datagen.duplicates(40, 3, 1)  # one distinct point: every weight 0 from the start
    seeds, pot = same_as_oracle(X, 5, datagen.uniforms53(okm.n_uniforms(5), 2), per_seed=per_seed)
    assert pot == 0


@pytest.mark.parametrize("per_seed", [False, True])
def test_kilosort4_seeding_section_full_size(per_seed):
    """The page's measured section: 1,416 points, 102 features, 200 seeds."""
    wl = datagen.make("ks4_seeding_1416x102")
    seeds, pot = same_as_oracle(wl["X"], wl["k"], wl["uniforms"], per_seed=per_seed)
    assert len(set(seeds)) == 200
    say("section seeding: potential %d, first seeds %s" % (pot, seeds[:6]))


def test_paths_agree_on_many_small_sections():
    """Both paths on 24 random small sections (no oracle: they must agree bit
    for bit, and each is checked against the oracle above)."""
    rng = np.random.default_rng(3)
    for t in range(24):
        n = int(rng.integers(1, 4097))
        d = int(rng.integers(1, 130))
        k = int(rng.integers(1, min(n, 300) + 1))
        X = datagen.gaussian_mixture(n, d, int(rng.integers(1, 30)), 100 + t)
        u = datagen.uniforms53(okm.n_uniforms(k), 200 + t)
        assert run_gpu(X, k, u) == run_gpu(X, k, u, per_seed=True), (n, d, k)


def test_repeatable_and_uniform_mask():
    wl = datagen.make("ks4_seeding_1416x102")
    X, k, u = wl["X"], 60, wl["uniforms"][:okm.n_uniforms(60)]
    a = run_gpu(X, k, u)
    b = run_gpu(X, k, u)
    assert a == b
    high = (np.asarray(u, np.uint64) | np.uint64(1 << 60)).astype(np.uint64)
    assert run_gpu(X, k, high) == a  # only the low 53 bits count


def test_bad_arguments():
    X = torch.zeros((4, 10), dtype=torch.float32, device="cuda")
    u = torch.zeros(3, dtype=torch.int64, device="cuda")
    with pytest.raises(binding.EkhError) as e:  # k = 5 needs 1 + 4 * 3 uniforms
        ekh.kmeanspp(X, 5, u)
    assert e.value.code == binding.EKH_EINVAL
    with pytest.raises(binding.EkhError):
        ekh.kmeanspp(X, 0, u)
    with pytest.raises(ValueError):
        ekh.kmeanspp(X, 1, u.float())
