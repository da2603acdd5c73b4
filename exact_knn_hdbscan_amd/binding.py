"""Thin ctypes binding of libekh.so (C ABI in include/ekh.h).

Argument marshalling only: every computation runs in the HIP library.  Point
sets are torch float32 CUDA tensors of shape [d, n] with unit stride along n
(feature-major, the layout of the clustering page); the leading dimension is
taken from ``stride(0)``.  Outputs and the workspace are allocated with torch on
the input's device and the work is enqueued on torch's current stream.

There is no fallback: if the library is missing or no GPU is present the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libekh.so")

EKH_OK = 0
EKH_EINVAL = -1
EKH_EWORKSPACE = -2
EKH_EHIP = -3
EKH_EINTERNAL = -4
MAX_K = 32
MAX_DIM = 256
MAX_ROUNDS = 64
MST_NO_NEIGHBOUR_EDGES = 1
MST_NO_COMPONENT_BOUND = 2

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_p = ctypes.c_void_p
_sz = ctypes.c_size_t


class MstStats(ctypes.Structure):
    _fields_ = [
        ("rounds", ctypes.c_int32),
        ("n_components", ctypes.c_int32 * MAX_ROUNDS),
        ("resolved", ctypes.c_int64 * MAX_ROUNDS),
        ("skipped", ctypes.c_int64 * MAX_ROUNDS),
        ("scanned", ctypes.c_int64 * MAX_ROUNDS),
        ("edges_added", ctypes.c_int64 * MAX_ROUNDS),
        ("round_ms", ctypes.c_double * MAX_ROUNDS),
        ("scanned_giant", ctypes.c_int64 * MAX_ROUNDS),
    ]

    def as_dict(self) -> dict:
        r = self.rounds
        return {
            "rounds": r,
            "n_components": list(self.n_components[:r]),
            "resolved": list(self.resolved[:r]),
            "skipped": list(self.skipped[:r]),
            "scanned": list(self.scanned[:r]),
            "edges_added": list(self.edges_added[:r]),
            "round_ms": list(self.round_ms[:r]),
            "scanned_giant": list(self.scanned_giant[:r]),
        }


class HdbscanInfo(ctypes.Structure):
    _fields_ = [("n_entries", ctypes.c_int64), ("n_clusters", ctypes.c_int32), ("n_selected", ctypes.c_int32)]


class EkhError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("ekh error %d: %s" % (code, msg))
        self.code = code


_lock = threading.Lock()
_lib = None


def library() -> ctypes.CDLL:
    """Loads libekh.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libekh.so is not built (run __graft_entry__.build())")
            lib = ctypes.CDLL(LIB_PATH)
            lib.ekh_version.restype = ctypes.c_int
            lib.ekh_last_error.restype = ctypes.c_char_p
            lib.ekh_knn_workspace_bytes.argtypes = [_i64, _i64, _i32, _i32, _i64]
            lib.ekh_knn_workspace_bytes.restype = _sz
            lib.ekh_knn.argtypes = [_p, _i64, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _i64, _p, _sz, _p]
            lib.ekh_knn_plan.argtypes = [_i64, _i64, _i32, _i32, _i64, ctypes.POINTER(_i64)]
            lib.ekh_knn_noalloc_bytes.argtypes = [_i64, _i64, _i32, _i32, _i64]
            lib.ekh_knn_noalloc_bytes.restype = _sz
            lib.ekh_knn_noalloc.argtypes = [_p, _i64, _i64, _p, _i64, _i64, _i32, _i32, _p, _p, _i64, _p]
            lib.ekh_core_workspace_bytes.argtypes = [_i64, _i32, _i32]
            lib.ekh_core_workspace_bytes.restype = _sz
            lib.ekh_core_distances.argtypes = [_p, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _sz, _p]
            lib.ekh_mst_workspace_bytes.argtypes = [_i64, _i32, _i32, ctypes.c_int]
            lib.ekh_mst_workspace_bytes.restype = _sz
            lib.ekh_mst_boruvka.argtypes = [_p, _i64, _i64, _i32, _p, _i32, _p, _p, _u32, _p, _p, _p, _p, _p, _sz,
                                            _p]
            lib.ekh_hdbscan_tail.argtypes = [_p, _p, _p, _i64, _i32, _p, _p, _p, _p, _p, _p, _p]
            lib.ekh_cluster_edge_counts.argtypes = [_p, _i64, _i32, _i64, _p, _p, _i32, _p, _p, _sz, _p]
            lib.ekh_merge_tree.argtypes = [_p, _i32, ctypes.c_double, _p, _p, _p]
            lib.ekh_bipartite_workspace_bytes.argtypes = [_i64, _i32]
            lib.ekh_bipartite_workspace_bytes.restype = _sz
            lib.ekh_bipartite_assign.argtypes = [_p, _i64, _i32, _i64, _i32, _p, ctypes.c_double, _i32, _p, _p, _p, _p,
                                                 _sz, _p]
            lib.ekh_kmeanspp_workspace_bytes.argtypes = [_i64, _i32, _u32]
            lib.ekh_kmeanspp_workspace_bytes.restype = _sz
            lib.ekh_kmeanspp.argtypes = [_p, _i64, _i64, _i32, _i32, _p, _i64, _u32, _p, _p, _p, _sz, _p]
            lib.ekh_timer_enable.argtypes = [ctypes.c_int]
            lib.ekh_timer_read.argtypes = [ctypes.c_int, ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(ctypes.c_double)]
            _lib = lib
    return _lib


def _check(rc: int):
    if rc != EKH_OK:
        raise EkhError(rc, library().ekh_last_error().decode(errors="replace"))


def _points(X: torch.Tensor, name: str):
    if not isinstance(X, torch.Tensor) or X.dtype != torch.float32 or X.dim() != 2:
        raise TypeError("%s must be a float32 tensor [d, n]" % name)
    if not X.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if X.stride(1) != 1 and X.shape[1] > 1:
        raise ValueError("%s must have unit stride along points" % name)
    ld = X.stride(0) if X.shape[0] > 1 else X.shape[1]
    return X.data_ptr(), int(ld), int(X.shape[1]), int(X.shape[0])


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _out(t, shape, dtype, dev, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != dev:
        raise ValueError("%s must be a contiguous %s tensor %s on %s" % (name, dtype, tuple(shape), dev))
    return t


def _workspace(nbytes: int, dev):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def knn_workspace_bytes(n: int, m: int, d: int, k: int, max_chunk_dots: int = 0) -> int:
    return int(library().ekh_knn_workspace_bytes(n, m, d, k, max_chunk_dots))


def knn_plan(n: int, m: int, d: int, k: int, max_chunk_dots: int = 0) -> dict:
    """Launch layout of the kNN tile kernel for these sizes (host only)."""
    out = (_i64 * 8)()
    _check(library().ekh_knn_plan(n, m, d, k, max_chunk_dots, out))
    keys = ("chunk_rows", "tile_rows", "body_tiles", "splits", "slots", "last_body_tiles", "last_splits",
            "chunks_in_flight")
    return dict(zip(keys, (int(v) for v in out)))


def core_workspace_bytes(n: int, d: int, min_samples: int) -> int:
    return int(library().ekh_core_workspace_bytes(n, d, min_samples))


def mst_workspace_bytes(n: int, d: int, min_samples: int, with_neighbours: bool = True) -> int:
    return int(library().ekh_mst_workspace_bytes(n, d, min_samples, 1 if with_neighbours else 0))


def knn(X: torch.Tensor, Y: torch.Tensor, k: int, max_chunk_dots: int = 0, workspace: torch.Tensor = None,
        out_idx: torch.Tensor = None, out_dist: torch.Tensor = None):
    """k nearest points of Y for every point of X.

    Returns ``(idx int32 [n, k], dist float32 [n, k])``; rows ascending under
    (squared distance, index).  Passing the same tensor as X and Y makes the set
    its own database (self pairs at distance 0).  A caller-owned ``workspace``
    (uint8, at least knn_workspace_bytes()) and outputs may be passed in; the
    library checks the workspace size itself.
    """
    lib = library()
    px, ldx, n, d = _points(X, "X")
    py, ldy, m, dy = _points(Y, "Y")
    if dy != d:
        raise ValueError("X and Y differ in dimension")
    if X.device != Y.device:
        raise ValueError("X and Y on different devices")
    idx = _out(out_idx, (n, k), torch.int32, X.device, "out_idx")
    dist = _out(out_dist, (n, k), torch.float32, X.device, "out_dist")
    ws = workspace if workspace is not None else _workspace(lib.ekh_knn_workspace_bytes(n, m, d, k, max_chunk_dots),
                                                            X.device)
    _check(lib.ekh_knn(px, ldx, n, py, ldy, m, d, k, idx.data_ptr(), dist.data_ptr(), max_chunk_dots,
                       ws.data_ptr(), ws.numel(), _stream(X.device)))
    return idx, dist


def knn_noalloc(X: torch.Tensor, Y: torch.Tensor, k: int, max_chunk_dots: int = 0, out_idx: torch.Tensor = None,
                out_dist: torch.Tensor = None):
    """ekh_knn_noalloc: knn() with the library's static scratch instead of a
    workspace (no allocation inside the call).  Outputs may be passed in
    (int32 / float32 [n, k] on X's device); otherwise they are allocated here."""
    lib = library()
    px, ldx, n, d = _points(X, "X")
    py, ldy, m, dy = _points(Y, "Y")
    if dy != d:
        raise ValueError("X and Y must have the same dimension")
    if out_idx is None:
        out_idx = torch.empty((n, k), dtype=torch.int32, device=X.device)
    if out_dist is None:
        out_dist = torch.empty((n, k), dtype=torch.float32, device=X.device)
    _check(lib.ekh_knn_noalloc(px, ldx, n, py, ldy, m, d, k, _ptr(out_idx), _ptr(out_dist), max_chunk_dots,
                               _stream(X.device)))
    return out_idx, out_dist


def core_distances(X: torch.Tensor, min_samples: int, return_neighbours: bool = False, workspace=None):
    """Core distances [n] (float32); with ``return_neighbours`` also the self-kNN
    rows ``(idx int32 [n, ms+1], d2 float32 [n, ms+1])``."""
    lib = library()
    px, ldx, n, d = _points(X, "X")
    core = torch.empty(n, dtype=torch.float32, device=X.device)
    nb_idx = nb_d2 = None
    if return_neighbours:
        nb_idx = torch.empty((n, min_samples + 1), dtype=torch.int32, device=X.device)
        nb_d2 = torch.empty((n, min_samples + 1), dtype=torch.float32, device=X.device)
    need = lib.ekh_core_workspace_bytes(n, d, min_samples)
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, X.device)
    _check(lib.ekh_core_distances(px, ldx, n, d, min_samples, core.data_ptr(), _ptr(nb_idx), _ptr(nb_d2),
                                  ws.data_ptr(), ws.numel(), _stream(X.device)))
    if return_neighbours:
        return core, nb_idx, nb_d2
    return core


def mst_boruvka(X: torch.Tensor, core: torch.Tensor, min_samples: int, nbr_idx: torch.Tensor = None,
                nbr_d2: torch.Tensor = None, flags: int = 0, return_stats: bool = False, workspace=None):
    """Minimum spanning tree of max(core_a, core_b, |a - b|).

    Returns ``(lo int32 [n-1], hi int32 [n-1], w float32 [n-1])`` sorted by
    (w, lo, hi), plus a stats dict if ``return_stats``.  Blocks until done.
    """
    lib = library()
    px, ldx, n, d = _points(X, "X")
    if core.dtype != torch.float32 or core.shape != (n,) or not core.is_contiguous() or core.device != X.device:
        raise ValueError("core must be a contiguous float32 [n] tensor on X's device")
    with_nb = nbr_idx is not None
    if with_nb:
        K = min_samples + 1
        for t, dt in ((nbr_idx, torch.int32), (nbr_d2, torch.float32)):
            if t is None or t.dtype != dt or t.shape != (n, K) or not t.is_contiguous():
                raise ValueError("neighbour rows must be contiguous [n, min_samples + 1] (int32, float32)")
    ne = max(n - 1, 0)
    lo = torch.empty(ne, dtype=torch.int32, device=X.device)
    hi = torch.empty(ne, dtype=torch.int32, device=X.device)
    w = torch.empty(ne, dtype=torch.float32, device=X.device)
    stats = MstStats()
    need = lib.ekh_mst_workspace_bytes(n, d, min_samples, 1 if with_nb else 0)
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, X.device)
    _check(lib.ekh_mst_boruvka(px, ldx, n, d, core.data_ptr(), min_samples, _ptr(nbr_idx), _ptr(nbr_d2), flags,
                               lo.data_ptr(), hi.data_ptr(), w.data_ptr(), ctypes.byref(stats), ws.data_ptr(),
                               ws.numel(), _stream(X.device)))
    if return_stats:
        return lo, hi, w, stats.as_dict()
    return lo, hi, w


def hdbscan_tail(lo, hi, w, min_cluster_size: int, return_tree: bool = False):
    """Cluster labels from a spanning tree (ekh_hdbscan_tail, host code).

    ``lo``, ``hi`` (int32) and ``w`` (float32) are the n - 1 tree edges, e.g.
    the outputs of mst_boruvka (torch tensors on any device, or numpy arrays;
    device tensors are copied to the host here).  Returns labels (numpy int32
    [n], -1 = noise); with ``return_tree`` also a dict with the condensed tree
    (parent, child, lambda, size), the stability of every cluster and the
    counts.
    """
    import numpy as np

    def host(a, dt):
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu").numpy()
        return np.ascontiguousarray(a, dtype=dt)

    lo, hi, w = host(lo, np.int32), host(hi, np.int32), host(w, np.float32)
    if not (lo.ndim == hi.ndim == w.ndim == 1 and lo.shape == hi.shape == w.shape):
        raise ValueError("lo, hi and w must be 1-D arrays of equal length")
    n = lo.shape[0] + 1
    labels = np.empty(n, np.int32)
    info = HdbscanInfo()
    if return_tree:
        par = np.empty(2 * n, np.int64)
        chi = np.empty(2 * n, np.int64)
        lam = np.empty(2 * n, np.float64)
        siz = np.empty(2 * n, np.int64)
        st = np.empty(n, np.float64)
        ptrs = [par.ctypes.data, chi.ctypes.data, lam.ctypes.data, siz.ctypes.data, st.ctypes.data]
    else:
        ptrs = [None] * 5
    _check(library().ekh_hdbscan_tail(lo.ctypes.data, hi.ctypes.data, w.ctypes.data, n, min_cluster_size,
                                      labels.ctypes.data, *ptrs, ctypes.byref(info)))
    if not return_tree:
        return labels
    ne, nc = info.n_entries, info.n_clusters
    return labels, {"parent": par[:ne], "child": chi[:ne], "lambda": lam[:ne], "size": siz[:ne],
                    "stability": st[:nc], "n_clusters": nc, "n_selected": info.n_selected}


def bipartite_workspace_bytes(m: int, n_clusters: int) -> int:
    return int(library().ekh_bipartite_workspace_bytes(m, n_clusters))


def bipartite_assign(nbr: torch.Tensor, m: int, n_clusters: int, init_right: torch.Tensor, gamma: float = 1.0,
                     max_rounds: int = 200, workspace: torch.Tensor = None):
    """Bipartite kNN-graph assignment (ekh_bipartite_assign).  nbr: int32 [n, k]
    on the GPU (row-major, each row a spike's neighbours among the m right
    nodes); init_right: int32 [m] labels in [0, n_clusters).  Returns (left
    labels [n], right labels [m], rounds run)."""
    if nbr.dtype != torch.int32 or nbr.dim() != 2 or not nbr.is_contiguous() or not nbr.is_cuda:
        raise ValueError("nbr must be a contiguous int32 [n, k] CUDA tensor")
    if init_right.dtype != torch.int32 or init_right.shape != (m,) or not init_right.is_cuda:
        raise ValueError("init_right must be an int32 [m] CUDA tensor")
    lib = library()
    n, k = nbr.shape
    dev = nbr.device
    left = torch.empty(n, dtype=torch.int32, device=dev)
    right = torch.empty(m, dtype=torch.int32, device=dev)
    ws = workspace if workspace is not None else _workspace(bipartite_workspace_bytes(m, n_clusters), dev)
    rounds = ctypes.c_int32(0)
    _check(lib.ekh_bipartite_assign(nbr.data_ptr(), n, k, m, n_clusters, init_right.contiguous().data_ptr(),
                                    float(gamma), max_rounds, left.data_ptr(), right.data_ptr(), ctypes.byref(rounds),
                                    ws.data_ptr(), ws.numel(), _stream(dev)))
    return left, right, int(rounds.value)


def cluster_edge_counts(nbr: torch.Tensor, left: torch.Tensor, right: torch.Tensor, n_clusters: int):
    """Edge counts between clusters (ekh_cluster_edge_counts): uint32-valued
    int64 tensor [C, C] on the GPU, counts[a, b] = edges (i, r) with left[i] = a
    and right[r] = b."""
    for t, name in ((nbr, "nbr"), (left, "left"), (right, "right")):
        if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(name + " must be a contiguous int32 CUDA tensor")
    n, k = nbr.shape
    m = right.shape[0]
    dev = nbr.device
    out = torch.empty((n_clusters, n_clusters), dtype=torch.int32, device=dev)
    ws = _workspace(256, dev)
    _check(library().ekh_cluster_edge_counts(nbr.data_ptr(), n, k, m, left.data_ptr(), right.data_ptr(), n_clusters,
                                             out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return out.to(torch.int64) & 0xFFFFFFFF


EKH_KMEANSPP_PER_SEED_LAUNCHES = 1


def kmeanspp_workspace_bytes(n: int, k: int, per_seed_launches: bool = False) -> int:
    return int(library().ekh_kmeanspp_workspace_bytes(n, k, EKH_KMEANSPP_PER_SEED_LAUNCHES if per_seed_launches
                                                       else 0))


def kmeanspp(X: torch.Tensor, k: int, uniforms: torch.Tensor, per_seed_launches: bool = False,
             workspace: torch.Tensor = None):
    """Greedy k-means++ seeding (ekh_kmeanspp) of the columns of X [d, n]
    (float32 on the GPU).  uniforms: int64 or uint64 CUDA tensor of at least
    1 + (k - 1) (2 + floor(ln k)) values in [0, 2^53).  per_seed_launches
    forces the two-launches-per-seed path (same results, less workspace).
    Returns (seeds int32 [k], potential int64 [1]), both on the GPU; nothing is
    read back."""
    Xp, ldx, n, d = _points(X, "X")
    if uniforms.dtype not in (torch.int64, torch.uint64) or uniforms.dim() != 1 or not uniforms.is_cuda \
            or not uniforms.is_contiguous():
        raise ValueError("uniforms must be a contiguous 1-D int64 or uint64 CUDA tensor")
    dev = X.device
    seeds = torch.empty(k, dtype=torch.int32, device=dev)
    pot = torch.empty(1, dtype=torch.int64, device=dev)
    flags = EKH_KMEANSPP_PER_SEED_LAUNCHES if per_seed_launches else 0
    ws = workspace if workspace is not None else _workspace(kmeanspp_workspace_bytes(n, k, per_seed_launches), dev)
    _check(library().ekh_kmeanspp(Xp, ldx, n, d, k, uniforms.data_ptr(), uniforms.numel(), flags, seeds.data_ptr(),
                                  pot.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev)))
    return seeds, pot


def merge_tree(counts, gamma: float = 1.0):
    """Merging tree of the clusters (ekh_merge_tree, host code): counts [C, C]
    (torch tensor on any device, or numpy; non-negative) -> list of (a, b, dQ)
    for the C - 1 merges."""
    import numpy as np

    if isinstance(counts, torch.Tensor):
        counts = counts.detach().to("cpu").numpy()
    c = np.ascontiguousarray(counts, dtype=np.uint32)
    C = c.shape[0]
    if c.shape != (C, C):
        raise ValueError("counts must be square")
    a = np.empty(max(C - 1, 0), np.int32)
    b = np.empty(max(C - 1, 0), np.int32)
    g = np.empty(max(C - 1, 0), np.float64)
    _check(library().ekh_merge_tree(c.ctypes.data, C, float(gamma), a.ctypes.data, b.ctypes.data, g.ctypes.data))
    return [(int(x), int(y), float(z)) for x, y, z in zip(a, b, g)]


class kernel_timer:
    """Context manager around ekh_timer_enable / ekh_timer_read: HIP events on
    the launch stream around every launch of the dense kernels (the kNN tile
    kernel, the Boruvka scan, the symmetric self-kNN kernel)."""

    KNN_TILE = 0
    SCAN_TILE = 1
    KNN_SYM = 2

    def __enter__(self):
        _check(library().ekh_timer_enable(1))
        return self

    def __exit__(self, *exc):
        return False

    def read(self, kernel_id: int) -> dict:
        n = _i64()
        ms = ctypes.c_double()
        fl = ctypes.c_double()
        _check(library().ekh_timer_read(kernel_id, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl)))
        return {"launches": n.value, "ms": ms.value, "flop": fl.value}

    @staticmethod
    def stop():
        library().ekh_timer_enable(0)

