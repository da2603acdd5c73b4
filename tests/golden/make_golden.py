"""Writes the float64 oracle's results for the full-size clip workloads.

Calls only the CPU oracle (oracle/) and the seeded generators.  For each
workload it writes:

* tests/golden/<workload>_oracle.json: the core-distance sum and quantiles,
  the tree's total weight and weight quantiles, and the oracle's HDBSCAN tail
  on its own tree (min_cluster_size 20): cluster count, noise count and sorted
  cluster sizes;
* tests/golden/<workload>_oracle_tree.npz (compressed): the oracle's core
  distances (float64 [n]) and its minimum spanning tree as int32 ``lo``, ``hi``
  ([n - 1], lo < hi), stored in (lo, hi) order so that they compress well.
  The edge weights are not stored: a test recomputes them in float64 with
  ``oracle.pair_weights`` from the stored core distances.

The GPU tests compare against these at full size, where running the oracle
inside a test would take too long (dense Prim over 500,000 points takes hours
on the host).

Usage: python tests/golden/make_golden.py clips_100000x61 [clips_500000x61 ...] [--threads N]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from exact_knn_hdbscan_amd import datagen  # noqa: E402
from oracle import hdbscan_tail  # noqa: E402

QS = [0.0, 0.01, 0.1, 0.25, 0.5, 0.75, 0.9, 0.99, 1.0]
MIN_CLUSTER_SIZE = 20  # the HDBSCAN page's results use min_cluster_size = 20


def summarize(name, threads):
    wl = datagen.make(name)
    X = wl["X"]
    ms = wl["min_samples"]
    t0 = time.time()
    core = oracle.core_distances(X, ms, nthreads=threads)
    t1 = time.time()
    print("%s: core distances %.0f s" % (name, t1 - t0), flush=True)
    lo, hi, w = oracle.mst_prim(X, core, nthreads=threads)
    t2 = time.time()
    print("%s: Prim %.0f s" % (name, t2 - t1), flush=True)
    lab = hdbscan_tail.hdbscan_tail(lo, hi, w, X.shape[1], MIN_CLUSTER_SIZE)["labels"]
    t3 = time.time()
    sizes = np.bincount(lab[lab >= 0]) if (lab >= 0).any() else np.zeros(0, np.int64)
    order = np.lexsort((hi, lo))
    tree = {"core": core.astype(np.float64), "lo": lo[order].astype(np.int32), "hi": hi[order].astype(np.int32)}
    summary = {
        "workload": name, "seed": 0, "min_samples": ms, "n": int(X.shape[1]), "d": int(X.shape[0]),
        "core_sum": float(core.sum()), "core_quantiles": [float(v) for v in np.quantile(core, QS)],
        "mst_total_weight": float(w.sum()), "mst_weight_quantiles": [float(v) for v in np.quantile(w, QS)],
        "quantile_levels": QS,
        "hdbscan_min_cluster_size": MIN_CLUSTER_SIZE, "hdbscan_n_clusters": int(len(sizes)),
        "hdbscan_noise": int((lab < 0).sum()), "hdbscan_cluster_sizes_sorted": sorted(int(v) for v in sizes),
        "oracle_seconds": {"core": t1 - t0, "prim": t2 - t1, "tail": t3 - t2,
                           "threads": threads or oracle.max_threads()},
        "tree_file": name + "_oracle_tree.npz",
        "source": "tests/golden/make_golden.py (float64 oracle: direct-difference kNN, dense Prim)",
    }
    return summary, tree


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--threads", type=int, default=0)
    a = ap.parse_args()
    for name in a.workloads:
        s, tree = summarize(name, a.threads)
        np.savez_compressed(os.path.join(HERE, name + "_oracle_tree.npz"), **tree)
        path = os.path.join(HERE, name + "_oracle.json")
        with open(path, "w") as f:
            json.dump(s, f, indent=1)
        print("wrote", path, s["oracle_seconds"], flush=True)


if __name__ == "__main__":
    main()
