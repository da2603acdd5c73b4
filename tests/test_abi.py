"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before any GPU
call (the pointers passed here are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ekh.h")
LIB = os.path.join(ROOT, "exact_knn_hdbscan_amd", "libekh.so")


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(ekh_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libekh.so not built")
    from exact_knn_hdbscan_amd import binding
    return binding.library()


def test_header_declares_the_three_entry_points():
    names = declared()
    for n in ("ekh_knn", "ekh_core_distances", "ekh_mst_boruvka"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared():
        assert hasattr(lib, name), name


def test_workspace_queries(lib):
    assert lib.ekh_knn_workspace_bytes(1000, 500, 61, 10, 0) > 0
    assert lib.ekh_knn_workspace_bytes(1000, 500, 300, 10, 0) == 0  # d beyond the maximum
    assert lib.ekh_core_workspace_bytes(500000, 61, 10) > 0
    a = lib.ekh_mst_workspace_bytes(100000, 61, 10, 1)
    b = lib.ekh_mst_workspace_bytes(100000, 61, 10, 0)
    assert 0 < a < b


def plan(lib, n, m, d, k, dots=0):
    out = (ctypes.c_int64 * 8)()
    rc = lib.ekh_knn_plan(n, m, d, k, dots, out)
    return rc, list(out)


def test_knn_plan_of_the_clip_and_section_workloads(lib):
    # clips 500,000 x 61, lists of K = 11: 3,907 query tiles of 128 rows, 768
    # workgroups resident (256 CUs x 3): five whole rounds unsplit, the 67 tiles
    # left over in 11 database splits (737 workgroups: one more round)
    assert plan(lib, 500000, 500000, 61, 11) == (0, [500000, 128, 3840, 11, 768, 3840, 11, 1])
    # clips 100,000 x 61: 782 tiles, one whole round + 14 tiles in 54 splits
    assert plan(lib, 100000, 100000, 61, 11) == (0, [100000, 128, 768, 54, 768, 768, 54, 1])
    # Kilosort4 section, 50,000 queries x 5,000 (d = 102, 64-row tiles): 782 tiles
    rc, p = plan(lib, 50000, 5000, 102, 10)
    assert rc == 0 and p[1] == 64 and p[2] == 768 and p[3] > 1
    # fewer tiles than one round: every tile in the same number of splits
    rc, p = plan(lib, 5000, 50000, 102, 10)
    assert rc == 0 and p[2] == 0 and p[3] > 1
    # wide section in chunks of 64e6 dots: 3,200-row chunks of 50 tiles, two in
    # flight, each with half of the 512 resident workgroups (two per CU at
    # d = 200): 5 database splits instead of the 10 one chunk alone would take;
    # the last chunk 1,600 rows
    rc, p = plan(lib, 200000, 20000, 200, 10, 64_000_000)
    assert rc == 0 and p[0] == 3200 and p[1] == 64 and p[7] == 2 and p[4] == 256 and p[2] == 0 and p[5] == 0
    assert p[3] == 5 and p[6] >= p[3]


K_LIST = (2, 4, 8, 10, 11, 16, 32)


def test_knn_plan_invariants_and_workspace(lib):
    rng = __import__("numpy").random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(1, 700_000))
        m = int(rng.integers(1, 600_000))
        d = int(rng.integers(1, 257))
        k = int(rng.integers(1, min(32, m) + 1))
        dots = int(rng.choice([0, 0, int(rng.integers(1, 10 ** 10))]))
        rc, p = plan(lib, n, m, d, k, dots)
        assert rc == 0
        rows, qt, body, splits, slots, lbody, lsplits, conc = p
        K = next(x for x in K_LIST if x >= k)
        tiles = -(-m // (16 if d > 224 else 32))
        nchunks = -(-n // rows)
        assert conc == min(2, nchunks) and slots * conc in range(511, 769) and rows >= 1
        assert qt in (64, 128) and rows == n or rows % qt == 0
        last = n % rows or rows
        for r, b, s in ((rows, body, splits), (last, lbody, lsplits)):
            q = -(-r // qt)
            assert b % slots == 0 and 0 <= b < q or b == 0
            assert 1 <= s <= max(1, min(1024, tiles // 4))
            if b:
                assert s > 1  # whole tiles only pay off when the rest is split
            # the split scratch fits the workspace (8-byte entries)
            if s > 1:
                assert lib.ekh_knn_workspace_bytes(n, m, d, k, dots) >= 8 * K * s * (r - b * qt) * conc
    assert plan(lib, 0, 10, 4, 1)[0] == -1
    assert plan(lib, 10, 10, 4, 11)[0] == -1
    assert plan(lib, 10, 10, 257, 1)[0] == -1
    assert lib.ekh_knn_plan(10, 10, 4, 1, 0, None) == -1


BOGUS = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("args,code", [
    (dict(n=0), -1), (dict(d=0), -1), (dict(d=257), -1), (dict(k=0), -1), (dict(k=33), -1),
    (dict(k=11, m=10), -1), (dict(ldx=99), -1), (dict(ldx=1 << 48), -1), (dict(ldy=1 << 48), -1),
    (dict(X=None), -1), (dict(ws_bytes=1), -2),
])
def test_knn_rejects_bad_arguments(lib, args, code):
    a = dict(X=BOGUS, ldx=100, n=100, Y=BOGUS, ldy=50, m=50, d=8, k=5, ws=BOGUS, ws_bytes=1 << 30)
    a.update(args)
    rc = lib.ekh_knn(a["X"], a["ldx"], a["n"], a["Y"], a["ldy"], a["m"], a["d"], a["k"], BOGUS, BOGUS, 0,
                     a["ws"], a["ws_bytes"], None)
    assert rc == code
    assert lib.ekh_last_error()


def test_core_and_mst_reject_bad_arguments(lib):
    assert lib.ekh_core_distances(BOGUS, 10, 10, 3, 10, BOGUS, None, None, BOGUS, 1 << 30, None) == -1  # ms >= n
    assert lib.ekh_core_distances(BOGUS, 10, 10, 3, 3, None, None, None, BOGUS, 1 << 30, None) == -1
    assert lib.ekh_core_distances(BOGUS, 10, 10, 3, 3, BOGUS, BOGUS, None, BOGUS, 1 << 30, None) == -1
    assert lib.ekh_mst_boruvka(BOGUS, 10, 10, 3, BOGUS, 3, None, None, 8, BOGUS, BOGUS, BOGUS, None, BOGUS,
                               1 << 30, None) == -1  # unknown flag
    assert lib.ekh_mst_boruvka(BOGUS, 10, 10, 3, None, 3, None, None, 0, BOGUS, BOGUS, BOGUS, None, BOGUS,
                               1 << 30, None) == -1
    assert lib.ekh_mst_boruvka(BOGUS, 10, 10, 3, BOGUS, 3, None, None, 0, BOGUS, BOGUS, BOGUS, None, BOGUS,
                               16, None) == -2
    assert lib.ekh_timer_read(7, None, None, None) == -1


def test_bipartite_rejects_bad_arguments(lib):
    f = lib.ekh_bipartite_assign
    ok = dict(nbr=BOGUS, n=10, k=3, m=5, C=4, init=BOGUS, gamma=1.0, rounds=200, ws=BOGUS, ws_bytes=1 << 30)
    for change in (dict(k=0), dict(k=33), dict(n=0), dict(m=0), dict(C=0), dict(gamma=-1.0), dict(rounds=0),
                   dict(nbr=None), dict(ws=None), dict(n=1 << 30, k=2)):
        a = dict(ok, **change)
        rc = f(a["nbr"], a["n"], a["k"], a["m"], a["C"], a["init"], a["gamma"], a["rounds"], BOGUS, BOGUS, None, a["ws"],
               a["ws_bytes"], None)
        assert rc == -1, change
    a = dict(ok, ws_bytes=16)
    assert f(a["nbr"], a["n"], a["k"], a["m"], a["C"], a["init"], a["gamma"], a["rounds"], BOGUS, BOGUS, None, a["ws"],
             a["ws_bytes"], None) == -2
    assert lib.ekh_bipartite_workspace_bytes(5000, 40) >= 4 * (5000 * 40)
    assert lib.ekh_bipartite_workspace_bytes(0, 40) == 0


def test_kmeanspp_rejects_bad_arguments(lib):
    f = lib.ekh_kmeanspp
    # k = 200 -> L = 7 candidates, 1 + 199 * 7 = 1394 uniforms
    ok = dict(X=BOGUS, ldx=1416, n=1416, d=102, k=200, u=BOGUS, nu=1394, fl=0, seeds=BOGUS, ws=BOGUS,
              ws_bytes=1 << 30)
    for change in (dict(X=None), dict(u=None), dict(seeds=None), dict(ws=None), dict(n=0), dict(n=(1 << 22) + 1),
                   dict(d=0), dict(d=8193), dict(ldx=1415), dict(ldx=1 << 25), dict(k=0), dict(k=(1 << 20) + 1),
                   dict(nu=1393), dict(fl=2)):
        a = dict(ok, **change)
        rc = f(a["X"], a["ldx"], a["n"], a["d"], a["k"], a["u"], a["nu"], a["fl"], a["seeds"], None, a["ws"],
               a["ws_bytes"], None)
        assert rc == -1, change
        assert lib.ekh_last_error()
    for fl in (0, 1):
        a = dict(ok, ws_bytes=64, fl=fl)
        assert f(a["X"], a["ldx"], a["n"], a["d"], a["k"], a["u"], a["nu"], a["fl"], a["seeds"], None, a["ws"],
                 a["ws_bytes"], None) == -2
    # the section fits the distance-matrix path (n^2 floats); forced per-seed launches need ~24 n bytes
    assert lib.ekh_kmeanspp_workspace_bytes(1416, 200, 0) >= 4 * 1416 * 1416
    assert 8 * 1416 * 8 <= lib.ekh_kmeanspp_workspace_bytes(1416, 200, 1) < 4 * 1416 * 1416
    assert lib.ekh_kmeanspp_workspace_bytes(100000, 200, 0) == lib.ekh_kmeanspp_workspace_bytes(100000, 200, 1)
    assert lib.ekh_kmeanspp_workspace_bytes(0, 200, 0) == 0
    assert lib.ekh_kmeanspp_workspace_bytes(1416, 0, 0) == 0
    assert lib.ekh_kmeanspp_workspace_bytes(1416, 200, 4) == 0


@pytest.mark.parametrize("args,code", [
    (dict(n=0), -1), (dict(d=257), -1), (dict(k=33), -1), (dict(ldx=1 << 48), -1), (dict(X=None), -1),
    # sizes whose scratch exceeds the static array: refused before any GPU call
    (dict(n=400000, ldx=400000, m=400000, ldy=400000, d=61, k=11), -2),
])
def test_knn_noalloc_rejects_bad_arguments(lib, args, code):
    lib.ekh_knn_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_void_p]
    a = dict(X=BOGUS, ldx=100, n=100, Y=BOGUS, ldy=50, m=50, d=8, k=5)
    a.update(args)
    rc = lib.ekh_knn_noalloc(a["X"], a["ldx"], a["n"], a["Y"], a["ldy"], a["m"], a["d"], a["k"], BOGUS, BOGUS, 0,
                             None)
    assert rc == code
    assert lib.ekh_last_error()


def test_knn_noalloc_scratch_sizes(lib):
    lib.ekh_knn_noalloc_bytes.restype = ctypes.c_size_t
    lib.ekh_knn_noalloc_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int64]
    # the two section workloads fit the 64 MiB array, a 500,000-point self-kNN does not
    assert 0 < lib.ekh_knn_noalloc_bytes(50000, 5000, 102, 10, 0) < (64 << 20)
    assert 0 < lib.ekh_knn_noalloc_bytes(200000, 20000, 200, 10, 64000000) < (64 << 20)
    assert lib.ekh_knn_noalloc_bytes(500000, 500000, 61, 11, 0) > (64 << 20)
