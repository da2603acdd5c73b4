"""ekh_knn_noalloc (scratch in the library's static device array, no
allocation inside the call) against ekh_knn (caller workspace): identical
indices and distances, bit for bit, on two calls in a row through the C ABI,
the second with a smaller input; sizes beyond the array are refused."""
import ctypes

import numpy as np
import pytest
import torch

import exact_knn_hdbscan_amd as ekh
from exact_knn_hdbscan_amd import binding, datagen
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def call_noalloc(X, Y, k, dots):
    """ekh_knn_noalloc through the C ABI (ctypes), outputs preallocated here."""
    lib = binding.library()
    d, n = X.shape
    m = Y.shape[1]
    idx = torch.full((n, k), -7, dtype=torch.int32, device=X.device)
    dist = torch.full((n, k), float("nan"), dtype=torch.float32, device=X.device)
    stream = torch.cuda.current_stream(X.device).cuda_stream
    rc = lib.ekh_knn_noalloc(X.data_ptr(), X.stride(0), n, Y.data_ptr(), Y.stride(0), m, d, k, idx.data_ptr(),
                             dist.data_ptr(), dots, stream)
    assert rc == 0, lib.ekh_last_error().decode()
    return host(idx), host(dist)


def test_knn_noalloc_matches_knn_twice():
    cases = [
        # a chunked call (several row chunks, split database tiles) ...
        ("ks4-like 20,000 x 2,000, d = 102, k = 10, chunks of 3,000 rows",
         datagen.gaussian_mixture(20000, 102, 40, seed=21), 2000, 10, 3000 * 2000),
        # ... then a smaller one with odd sizes
        ("3,001 x 777, d = 61, k = 7", datagen.spike_clips(3001, 6, seed=22), 777, 7, 0),
    ]
    for label, P, m, k, dots in cases:
        X = dev(P)
        Y = dev(np.ascontiguousarray(P[:, ::P.shape[1] // m][:, :m]))
        need = ekh.library().ekh_knn_noalloc_bytes(X.shape[1], m, X.shape[0], k, dots)
        say("knn_noalloc %s (scratch %d bytes)" % (label, need))
        assert 0 < need <= (64 << 20)
        gi, gd = call_noalloc(X, Y, k, dots)
        ri, rd = ekh.knn(X, Y, k, max_chunk_dots=dots)
        np.testing.assert_array_equal(gi, host(ri))
        np.testing.assert_array_equal(gd.view(np.uint32), host(rd).view(np.uint32))


def test_knn_noalloc_refuses_sizes_beyond_its_scratch():
    lib = ekh.library()
    n, m, d = 400000, 400000, 61
    need = lib.ekh_knn_noalloc_bytes(n, m, d, 11, 0)
    assert need > (64 << 20)
    # refused on the host, before any GPU work (the pointers are never used)
    X = torch.empty((1, 1), dtype=torch.float32, device="cuda:0")
    rc = lib.ekh_knn_noalloc(X.data_ptr(), n, n, X.data_ptr(), m, m, d, 11, X.data_ptr(), X.data_ptr(), 0,
                             torch.cuda.current_stream().cuda_stream)
    assert rc == -2 and b"static scratch" in lib.ekh_last_error()
