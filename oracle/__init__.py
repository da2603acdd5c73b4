"""CPU oracle (float64) for exact kNN, core distances and the mutual-reachability MST.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may use this package; the product path never imports it.  It shares
no code with the HIP library.  The arithmetic lives in ``oracle.c`` (plain
float64 loops, see its header for the definitions and their sources on the
pages); this module compiles it with gcc when needed and marshals numpy arrays.

Every function takes feature-major float32 point sets ``[d, n]`` (element (f, i)
at ``X[f, i]``), the layout of the clustering page ("k-nearest neighbours are a
matrix product").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_p = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2 -fopenmp)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            lib.orc_knn.argtypes = [_p, _i64, _i64, _p, _i64, _i64, _int, _int, _p, _p, _int]
            lib.orc_core_distances.argtypes = [_p, _i64, _i64, _int, _int, _p, _int]
            lib.orc_prim.argtypes = [_p, _i64, _i64, _int, _p, _p, _p, _p, _int]
            lib.orc_kruskal.argtypes = [_p, _i64, _i64, _int, _p, _p, _p, _p]
            lib.orc_pair_weights.argtypes = [_p, _i64, _int, _p, _i64, _p, _p, _p, _p, _int]
            lib.orc_sqdist.argtypes = [_p, _i64, _i64, _p, _i64, _i64, _int]
            lib.orc_sqdist.restype = ctypes.c_double
            lib.orc_max_threads.restype = _int
            _lib = lib
    return _lib


def _fm(X: np.ndarray) -> np.ndarray:
    X = np.asarray(X)
    if X.dtype != np.float32 or X.ndim != 2:
        raise TypeError("point sets are float32 [d, n]")
    return np.ascontiguousarray(X)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_p)


def max_threads() -> int:
    return int(_load().orc_max_threads())


def knn(X: np.ndarray, Y: np.ndarray, k: int, nthreads: int = 0):
    """k nearest points of Y (indices into Y) for every point of X.

    Returns ``(idx int32 [n, k], d2 float64 [n, k])``, each row ascending under
    (squared distance, index).  When Y is X the point itself is a candidate.
    """
    X = _fm(X)
    Y = _fm(Y)
    d, n = X.shape
    if Y.shape[0] != d:
        raise ValueError("dimension mismatch")
    m = Y.shape[1]
    idx = np.empty((n, k), np.int32)
    d2 = np.empty((n, k), np.float64)
    rc = _load().orc_knn(_ptr(X), n, n, _ptr(Y), m, m, d, k, _ptr(idx), _ptr(d2), nthreads)
    if rc:
        raise ValueError("orc_knn failed (%d)" % rc)
    return idx, d2


def core_distances(X: np.ndarray, min_samples: int, nthreads: int = 0) -> np.ndarray:
    """Distance of every point to its min_samples-th nearest point, itself included."""
    X = _fm(X)
    d, n = X.shape
    core = np.empty(n, np.float64)
    rc = _load().orc_core_distances(_ptr(X), n, n, d, min_samples, _ptr(core), nthreads)
    if rc:
        raise ValueError("orc_core_distances failed (%d)" % rc)
    return core


def _sort_edges(lo, hi, w):
    order = np.lexsort((hi, lo, w))  # primary key w, then lo, then hi
    return lo[order], hi[order], w[order]


def mst_prim(X: np.ndarray, core: np.ndarray, nthreads: int = 0):
    """Minimum spanning tree of max(core_a, core_b, |a - b|) by dense Prim.

    Returns ``(lo int32, hi int32, w float64)``, n-1 edges with lo < hi, sorted
    by (w, lo, hi).
    """
    X = _fm(X)
    d, n = X.shape
    core = np.ascontiguousarray(core, np.float64)
    lo = np.empty(max(n - 1, 0), np.int32)
    hi = np.empty(max(n - 1, 0), np.int32)
    w = np.empty(max(n - 1, 0), np.float64)
    rc = _load().orc_prim(_ptr(X), n, n, d, _ptr(core), _ptr(lo), _ptr(hi), _ptr(w), nthreads)
    if rc:
        raise ValueError("orc_prim failed (%d)" % rc)
    return _sort_edges(lo, hi, w)


def mst_kruskal(X: np.ndarray, core: np.ndarray):
    """The same tree by Kruskal over all n(n-1)/2 edges (n <= 20,000)."""
    X = _fm(X)
    d, n = X.shape
    core = np.ascontiguousarray(core, np.float64)
    lo = np.empty(max(n - 1, 0), np.int32)
    hi = np.empty(max(n - 1, 0), np.int32)
    w = np.empty(max(n - 1, 0), np.float64)
    rc = _load().orc_kruskal(_ptr(X), n, n, d, _ptr(core), _ptr(lo), _ptr(hi), _ptr(w))
    if rc:
        raise ValueError("orc_kruskal failed (%d)" % rc)
    return _sort_edges(lo, hi, w)


def pair_weights(X: np.ndarray, core: np.ndarray, a: np.ndarray, b: np.ndarray, nthreads: int = 0):
    """float64 (W(a_t, b_t), D(a_t, b_t)) for listed pairs."""
    X = _fm(X)
    d, n = X.shape
    core = np.ascontiguousarray(core, np.float64)
    a = np.ascontiguousarray(a, np.int32)
    b = np.ascontiguousarray(b, np.int32)
    w = np.empty(a.shape[0], np.float64)
    dist = np.empty(a.shape[0], np.float64)
    _load().orc_pair_weights(_ptr(X), n, d, _ptr(core), a.shape[0], _ptr(a), _ptr(b), _ptr(w), _ptr(dist),
                             nthreads)
    return w, dist


def sqdist(X: np.ndarray, i: int, Y: np.ndarray, j: int) -> float:
    X = _fm(X)
    Y = _fm(Y)
    return float(_load().orc_sqdist(_ptr(X), X.shape[1], i, _ptr(Y), Y.shape[1], j, X.shape[0]))


def mutual_reachability_matrix(X: np.ndarray, core: np.ndarray) -> np.ndarray:
    """Dense float64 n x n matrix of W (small n only; diagonal 0)."""
    X = _fm(X)
    n = X.shape[1]
    a, b = np.triu_indices(n, 1)
    w, _ = pair_weights(X, core, a.astype(np.int32), b.astype(np.int32))
    M = np.zeros((n, n))
    M[a, b] = w
    M[b, a] = w
    return M
