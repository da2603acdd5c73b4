"""Writes float64 oracle summaries of the full-size clip workloads.

Calls only the CPU oracle (oracle/) and the seeded generators.  For each
workload it stores, in tests/golden/<workload>_oracle.json: the core-distance
sum and quantiles, the MST's total weight, weight quantiles and a hash of its
edge list (sorted by (w, lo, hi)), and the oracle's HDBSCAN tail on that tree
(min_cluster_size 20): cluster count, noise count and sorted cluster sizes.
The GPU tests compare against these at full size, where running the oracle
inside a test would take too long.

Usage: python tests/golden/make_golden.py clips_100000x61 [clips_500000x61 ...] [--threads N]
"""
import argparse
import hashlib
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
    lo, hi, w = oracle.mst_prim(X, core, nthreads=threads)
    t2 = time.time()
    h = hashlib.sha256(np.stack([lo, hi]).astype(np.int32).tobytes()).hexdigest()
    lab = hdbscan_tail.hdbscan_tail(lo, hi, w, X.shape[1], MIN_CLUSTER_SIZE)["labels"]
    t3 = time.time()
    sizes = np.bincount(lab[lab >= 0]) if (lab >= 0).any() else np.zeros(0, np.int64)
    return {
        "workload": name, "seed": 0, "min_samples": ms, "n": int(X.shape[1]), "d": int(X.shape[0]),
        "core_sum": float(core.sum()), "core_quantiles": [float(v) for v in np.quantile(core, QS)],
        "mst_total_weight": float(w.sum()), "mst_weight_quantiles": [float(v) for v in np.quantile(w, QS)],
        "mst_edges_sha256": h, "quantile_levels": QS,
        "hdbscan_min_cluster_size": MIN_CLUSTER_SIZE, "hdbscan_n_clusters": int(len(sizes)),
        "hdbscan_noise": int((lab < 0).sum()), "hdbscan_cluster_sizes_sorted": sorted(int(v) for v in sizes),
        "oracle_seconds": {"core": t1 - t0, "prim": t2 - t1, "tail": t3 - t2,
                           "threads": threads or oracle.max_threads()},
        "source": "tests/golden/make_golden.py (float64 oracle: direct-difference kNN, dense Prim)",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--threads", type=int, default=0)
    a = ap.parse_args()
    for name in a.workloads:
        s = summarize(name, a.threads)
        path = os.path.join(HERE, name + "_oracle.json")
        with open(path, "w") as f:
            json.dump(s, f, indent=1)
        print("wrote", path, s["oracle_seconds"], flush=True)


if __name__ == "__main__":
    main()
