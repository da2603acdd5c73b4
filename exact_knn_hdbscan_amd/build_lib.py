"""Builds libekh.so (the HIP library) in-tree with hipcc for gfx950.

Each source under csrc/ is compiled to an object in csrc/_build/ (in parallel),
then linked into exact_knn_hdbscan_amd/libekh.so.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libekh.so")
# (source, object name, extra flags); the kNN kernels are instantiated once per list length
KNN_KS = [2, 4, 8, 10, 11, 16, 32]
SOURCES = [("tile_kernels.hip", "tile_kernels", []), ("boruvka_kernels.hip", "boruvka_kernels", []),
           ("api.hip", "api", []), ("bipartite.hip", "bipartite", []),
           ("kmeanspp.hip", "kmeanspp", ["-ffp-contract=off"])] + [("knn_inst.hip", "knn_k%d" % k, ["-DEKH_KNN_K=%d" % k]) for k in KNN_KS]
# host-only C++ (no device code), built with g++; -ffp-contract=off keeps every
# float64 expression as written (no fused multiply-adds)
HOST_SOURCES = [("hdbscan_tail.cpp", "hdbscan_tail"), ("merge_tree.cpp", "merge_tree")]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_*_f32 in generated code.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(job) -> str:
    src, name, extra = job
    obj = os.path.join(BUILD, name + ".o")
    if src.endswith(".cpp"):
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off", "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [hipcc()] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed for %s:\n%s" % (src, r.stderr[-6000:]))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), max(2, os.cpu_count() or 2))) as ex:
        objs = list(ex.map(_compile, SOURCES + [(src, name, []) for src, name in HOST_SOURCES]))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-4000:])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
