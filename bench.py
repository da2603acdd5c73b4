"""Benchmark of the hot path: exact self-kNN -> core distances -> Boruvka MST.

One step is one pass of the whole path over the 500,000 x 61 spike-clip set
(min_samples = 10): ekh_core_distances (exact self-kNN with K = 11 on MFMA,
every pair computed once: a bound pass against every 16th point, then the
symmetric pass; core distance = entry 10) followed by ekh_mst_boruvka (all
rounds, with the exact shortcuts, edges sorted).  Inputs are resident in HBM
before the timed region.

Prints one JSON line.  ``value`` is distance pairs (n^2, the ordered pairs the
exact self-kNN resolves) per second of the WHOLE step; the kNN-only rate, MST
time and the roofline of the dominant kernel (its algorithmic flop: 2 d per
pair it computes) are reported beside it, and so is
the host HDBSCAN tail (condensed tree, excess of mass, labels) on the last
step's tree, which is not part of the step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "kNN pair-distances/s + Borůvka MST time at 500k×61; % fp32 MFMA peak"
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X published dense fp32 matrix peak
COPY_BYTES = 1 << 30  # size of the calibration copy of --pmc-probe
SECTION_WARM_S = 0.5  # seconds of repeated section calls before they are timed
HBM_PEAK_GBS = 8000.0
TAIL_MIN_CLUSTER_SIZE = 20  # the HDBSCAN page's results use min_cluster_size = 20


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "knn_sym_traffic_clips_500000x61.md")
# the kernel and the planner that decides its launch layout
KNN_SOURCES = ["exact_knn_hdbscan_amd/csrc/tile_common.h", "exact_knn_hdbscan_amd/csrc/knn_inst.hip",
               "exact_knn_hdbscan_amd/csrc/ekh_internal.h", "exact_knn_hdbscan_amd/csrc/api.hip"]


def stored_traffic():
    """L2-miss (fabric) bytes per launch of the symmetric kNN kernel from the
    committed counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known
    size), or None if the kernel or planner sources have changed since the
    counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in KNN_SOURCES)).hexdigest()
    except OSError:
        return None
    m_t = re.search(r"^traffic_bytes_per_launch: (\d+)", text, re.M)
    m_h = re.search(r"^kernel_source_sha256: ([0-9a-f]+)", text, re.M)
    if not m_t or not m_h or m_h.group(1) != h:
        return None
    return int(m_t.group(1))


def cpu_baseline(X, k, budget_s=15.0):
    """The oracle (float64 C, all host threads) on a bounded sample of the same
    workload: exact k-NN of the first rows against all n points, in batches of
    64 rows until ~budget_s seconds have been spent."""
    import numpy as np

    import oracle

    n = X.shape[1]
    rows = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s and rows < n:
        b = min(64, n - rows)
        oracle.knn(np.ascontiguousarray(X[:, rows:rows + b]), X, k)
        rows += b
    dt = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": rows * n / dt,
        "unit": "pairs/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": "float64 exact %d-NN of the first %d of %d points against all %d (%.1f s)" % (k, rows, n, n, dt),
        "cpu_model": model,
    }


def time_bipartite(ekh, datagen, idx, m, oracle_too, n_clusters=40, reps=5):
    """ekh_bipartite_assign on the section's kNN graph (every spike's 10 nearest
    subset points), 40 starting labels drawn uniformly: median time per call,
    rounds, and (with the CPU baseline) the oracle on the same graph."""
    import numpy as np
    import torch

    init = torch.from_numpy(datagen.random_labels(m, n_clusters, 0)).cuda()
    ws = torch.empty(ekh.bipartite_workspace_bytes(m, n_clusters), dtype=torch.uint8, device=idx.device)
    ekh.bipartite_assign(idx, m, n_clusters, init, workspace=ws)
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        left, right, rounds = ekh.bipartite_assign(idx, m, n_clusters, init, workspace=ws)
        torch.cuda.synchronize()
        ts.append(1000.0 * (time.perf_counter() - t0))
    ms_call = float(np.median(ts))
    # edge counts between clusters (device; one warm-up call, then the median of reps) and the merging tree (host)
    counts = ekh.cluster_edge_counts(idx, left, right, n_clusters)
    tc = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        counts = ekh.cluster_edge_counts(idx, left, right, n_clusters)
        torch.cuda.synchronize()
        tc.append(1000.0 * (time.perf_counter() - t0))
    # the merging tree: host code on the counts in host memory (one warm-up call, then the median of reps)
    counts_h = counts.cpu().numpy()
    tree = ekh.merge_tree(counts_h)
    tm = []
    for _ in range(reps):
        t1 = time.perf_counter()
        tree = ekh.merge_tree(counts_h)
        tm.append(1000.0 * (time.perf_counter() - t1))
    res = {"ms": ms_call, "rounds": rounds,
           "edge_counts_ms": float(np.median(tc)), "merge_tree_ms": float(np.median(tm)), "merges": len(tree),
           "ms_per_round": ms_call / rounds, "n": int(idx.shape[0]), "m": m,
           "k": int(idx.shape[1]), "n_clusters": n_clusters, "labels_in_use": int(torch.unique(left).numel()),
           "where": "device, one 4-byte read-back per round (host clock around the call)"}
    if oracle_too:
        from oracle import bipartite as obip
        t0 = time.perf_counter()
        obip.assign(idx.cpu().numpy(), m, n_clusters, init.cpu().numpy())
        res["oracle_ms"] = 1000.0 * (time.perf_counter() - t0)
    return res


def time_seeding(ekh, datagen, oracle_too, reps=10):
    """ekh_kmeanspp on the page's seeding section (1,416 points, 102 features,
    200 seeds, 7 candidates each): median time per call on the host clock
    (launch cost included) and on stream events, for the library's default
    path (distance matrix + one seeding block) and for the path with two
    launches per seed, and (with the CPU baseline) the oracle on the same
    section, whose seeds must agree."""
    import numpy as np
    import torch

    wl = datagen.make("ks4_seeding_1416x102")
    X = torch.from_numpy(wl["X"]).cuda()
    u = torch.from_numpy(wl["uniforms"].astype(np.int64)).cuda()
    k = wl["k"]
    res = {"n": int(X.shape[1]), "d": int(X.shape[0]), "seeds": k,
           "where": "device, no host sync inside the call (host clock around call + sync)"}
    for key, per_seed in (("", False), ("per_seed_launches_", True)):
        ws = torch.empty(ekh.kmeanspp_workspace_bytes(X.shape[1], k, per_seed), dtype=torch.uint8, device=X.device)
        seeds, pot = ekh.kmeanspp(X, k, u, per_seed_launches=per_seed, workspace=ws)
        torch.cuda.synchronize()
        wall, gpu = [], []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record()
            seeds, pot = ekh.kmeanspp(X, k, u, per_seed_launches=per_seed, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            wall.append(1000.0 * (time.perf_counter() - t0))
            gpu.append(e0.elapsed_time(e1))
        res[key + "ms"] = float(np.median(wall))
        res[key + "stream_ms"] = float(np.median(gpu))
        res[key + "launches"] = 2 * k if per_seed else 2
        if not per_seed:
            got = (seeds.cpu().numpy().tolist(), int(pot.item()))
        else:
            res["paths_agree"] = got == (seeds.cpu().numpy().tolist(), int(pot.item()))
    if oracle_too:
        from oracle import kmeanspp as okm
        t0 = time.perf_counter()
        want = okm.seed(wl["X"], k, wl["uniforms"])
        res["oracle_ms"] = 1000.0 * (time.perf_counter() - t0)
        res["matches_oracle"] = got == (want[0], want[1])
    return res


def time_clips(ekh, datagen, oracle_too, reps=5):
    """The path (core distances + Boruvka MST) on the two other clip-like
    workloads: the tiny set (2,000 x 60) and clips 100,000 x 61, median of reps
    steps, with the kNN kernel's rate and the MST time.  With the CPU baseline,
    the oracle's core distances and Prim on the tiny set are timed beside the
    GPU (all host threads), and the stored oracle times of the two clip sets
    (tests/golden, written by make_golden.py) are quoted as context."""
    import numpy as np
    import torch

    out = {}
    for name in ("tiny_2000x60", "clips_100000x61"):
        wl = datagen.make(name)
        Xh = wl["X"]
        d, n = Xh.shape
        ms = wl.get("min_samples", 10)
        X = torch.from_numpy(Xh).cuda()
        wc = torch.empty(ekh.core_workspace_bytes(n, d, ms), dtype=torch.uint8, device=X.device)
        wm = torch.empty(ekh.mst_workspace_bytes(n, d, ms, True), dtype=torch.uint8, device=X.device)

        def step():
            core, ni, nd2 = ekh.core_distances(X, ms, return_neighbours=True, workspace=wc)
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            r = ekh.mst_boruvka(X, core, ms, ni, nd2, return_stats=True, workspace=wm)
            return r, e

        step()
        torch.cuda.synchronize()
        tot, knn = [], []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record()
            (lo, hi, w, st), ek = step()
            e1.record()
            torch.cuda.synchronize()
            tot.append(1000.0 * (time.perf_counter() - t0))
            knn.append(e0.elapsed_time(ek))
        # the tile kernel's launch durations, from more steps with the library's timer on
        timer = ekh.kernel_timer()
        timer.__enter__()
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        tk = timer.read(timer.KNN_TILE)
        tsym = timer.read(timer.KNN_SYM)
        timer.stop()
        ms_step, ms_knn = float(np.median(tot)), float(np.median(knn))
        pairs = float(n) * float(n)
        # the kNN kernels' rate over the pairs they compute (the symmetric pass
        # and its bound pass from 16,384 points on, else the tile kernel alone)
        kms = tk["ms"] + tsym["ms"]
        tfl = (tk["flop"] + tsym["flop"]) / (kms / 1e3) / 1e12 if kms else None
        res = {"n": n, "d": d, "min_samples": ms, "ms_per_step": ms_step, "knn_ms": ms_knn,
               "pairs_per_s": pairs / (ms_step / 1e3), "knn_pairs_per_s": pairs / (ms_knn / 1e3),
               "knn_kernel_tflops": tfl, "knn_kernel_frac": tfl / PEAK_FP32_MFMA_TFLOPS if tfl else None,
               "mst_ms": ms_step - ms_knn, "rounds": st["rounds"], "scanned": st["scanned"]}
        if oracle_too:
            import oracle
            if n <= 5000:
                t0 = time.perf_counter()
                core_o = oracle.core_distances(Xh, ms)
                t1 = time.perf_counter()
                oracle.mst_prim(Xh, core_o)
                t2 = time.perf_counter()
                res["oracle"] = {"core_ms": 1000.0 * (t1 - t0), "prim_ms": 1000.0 * (t2 - t1),
                                 "threads": oracle.max_threads()}
            g = os.path.join(ROOT, "tests", "golden", name + "_oracle.json")
            if os.path.exists(g):
                res["oracle_stored_seconds"] = json.load(open(g)).get("oracle_seconds")
        out[name] = res
        del X, wc, wm
    return out


def time_sections(ekh, datagen, oracle_too=False, reps=9):
    """ekh_knn on the two section workloads (50,000 x 5,000 at d = 102, k = 10; and
    200,000 x 20,000 at d = 200, k = 10, in chunks of max_chunk_dots = 64e6): median
    time per call with inputs resident, after SECTION_WARM_S of the same call, the
    tile kernel's rate per launch, the rate over the whole call, and the pair rate."""
    import numpy as np
    import torch

    out = {}
    for name in ("ks4_section_50000x102", "wide_section_200000x200"):
        wl = datagen.make(name)
        X, Y, k = torch.from_numpy(wl["X"]).cuda(), torch.from_numpy(wl["Y"]).cuda(), wl["k"]
        dots = wl.get("max_chunk_bytes", 0) // 4
        ws = torch.empty(ekh.knn_workspace_bytes(X.shape[1], Y.shape[1], X.shape[0], k, dots), dtype=torch.uint8,
                         device=X.device)
        # outputs and workspace allocated once, as a caller that repeats the call would
        oi = torch.empty((X.shape[1], k), dtype=torch.int32, device=X.device)
        od = torch.empty((X.shape[1], k), dtype=torch.float32, device=X.device)
        ekh.knn(X, Y, k, max_chunk_dots=dots, workspace=ws, out_idx=oi, out_dist=od)
        torch.cuda.synchronize()
        # steady state first: the same call repeated for SECTION_WARM_S (after
        # idle, or after other work, the first calls of a short kernel run at
        # lower clocks)
        t_end = time.perf_counter() + SECTION_WARM_S
        while time.perf_counter() < t_end:
            ekh.knn(X, Y, k, max_chunk_dots=dots, workspace=ws, out_idx=oi, out_dist=od)
            torch.cuda.synchronize()
        # the calls are timed with the library's kernel timer off; the tile
        # launches' own durations come from a second set of calls with it on
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ekh.knn(X, Y, k, max_chunk_dots=dots, workspace=ws, out_idx=oi, out_dist=od)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        timer = ekh.kernel_timer()
        timer.__enter__()
        for _ in range(reps):
            ekh.knn(X, Y, k, max_chunk_dots=dots, workspace=ws)
        torch.cuda.synchronize()
        tk = timer.read(timer.KNN_TILE)
        timer.stop()
        ms_call = float(np.median(ts))
        pairs = float(X.shape[1]) * float(Y.shape[1])
        plan = ekh.knn_plan(X.shape[1], Y.shape[1], X.shape[0], k, dots)
        # with two chunks in flight the tile launches overlap: tile_ms sums their
        # durations (each launch's own rate is tile_tflops); call_tflops is the
        # algorithmic flop of the whole call over its wall time
        out[name] = {"ms": ms_call, "pairs_per_s": pairs / (ms_call / 1e3), "k": k, "max_chunk_dots": dots,
                     "chunks_in_flight": plan["chunks_in_flight"],
                     "tile_launches": tk["launches"] // reps, "tile_ms": tk["ms"] / reps,
                     "tile_tflops": tk["flop"] / (tk["ms"] / 1e3) / 1e12 if tk["ms"] else None,
                     "call_tflops": 2.0 * X.shape[0] * pairs / (ms_call / 1e3) / 1e12}
        if name == "ks4_section_50000x102":
            idx, _ = ekh.knn(X, Y, k, workspace=ws)
            out["bipartite_assignment"] = time_bipartite(ekh, datagen, idx, Y.shape[1], oracle_too)
        del X, Y, ws
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="clips_500000x61")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sections", action="store_true", help="skip the ekh_knn section workloads")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for counter runs: one plain copy of COPY_BYTES (calibration), one pass of the path, and "
                         "(unless --no-sections) one ekh_knn call on each section workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_knn_hdbscan_amd as ekh
    from exact_knn_hdbscan_amd import datagen

    wl = datagen.make(args.workload)
    X = wl["X"]
    d, n = X.shape
    ms = wl.get("min_samples", 10)
    dev = torch.device("cuda:0")
    Xg = torch.from_numpy(X).to(dev)
    ws_core = torch.empty(ekh.core_workspace_bytes(n, d, ms), dtype=torch.uint8, device=dev)
    ws_mst = torch.empty(ekh.mst_workspace_bytes(n, d, ms, True), dtype=torch.uint8, device=dev)

    def step():
        core, ni, nd2 = ekh.core_distances(Xg, ms, return_neighbours=True, workspace=ws_core)
        t_knn_end = torch.cuda.Event(enable_timing=True)
        t_knn_end.record()
        out = ekh.mst_boruvka(Xg, core, ms, ni, nd2, return_stats=True, workspace=ws_mst)
        return out, t_knn_end

    if args.pmc_probe:
        # calibration: a device-to-device copy that reads and writes COPY_BYTES each
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        step()
        torch.cuda.synchronize()
        print("pmc probe: copy of %d bytes, one pass of %s" % (COPY_BYTES, args.workload), flush=True)
        if not args.no_sections:
            # one ekh_knn call on each section workload (their kernels in the same counter run)
            for name in ("ks4_section_50000x102", "wide_section_200000x200"):
                swl = datagen.make(name)
                Xs, Ys = torch.from_numpy(swl["X"]).to(dev), torch.from_numpy(swl["Y"]).to(dev)
                ekh.knn(Xs, Ys, swl["k"], max_chunk_dots=swl.get("max_chunk_bytes", 0) // 4)
                torch.cuda.synchronize()
                print("pmc probe: one ekh_knn call on %s" % name, flush=True)
                del Xs, Ys
        print("pmc probe done", flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    timer = ekh.kernel_timer()
    timer.__enter__()
    stats = None
    knn_ms = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        s0 = torch.cuda.Event(enable_timing=True)
        s0.record()
        (lo, hi, w, stats), e_knn = step()
        torch.cuda.synchronize()
        knn_ms.append(s0.elapsed_time(e_knn))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    total_s = t1 - t0
    ms_step = 1000.0 * total_s / args.steps
    tk = timer.read(timer.KNN_TILE)
    ts = timer.read(timer.SCAN_TILE)
    tsym = timer.read(timer.KNN_SYM)
    timer.stop()

    pairs = float(n) * float(n)
    value = pairs / (total_s / args.steps)
    dom_name, dom = max((("knn_sym_kernel", tsym), ("knn_tile_kernel", tk), ("scan_tile_kernel", ts)),
                        key=lambda kv: kv[1]["ms"])
    achieved = dom["flop"] / (dom["ms"] / 1e3) / 1e12 if dom["ms"] > 0 else 0.0
    knn_step_ms = float(np.median(knn_ms))
    mst_step_ms = ms_step - knn_step_ms
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n": n, "d": d, "min_samples": ms, "k": ms + 1,
                   "step": "core_distances(self-kNN K=11) + mst_boruvka (all rounds, shortcuts on)"},
        "knn": {"ms": knn_step_ms, "pairs_per_s": pairs / (knn_step_ms / 1e3),
                "sym_kernel_ms_per_step": tsym["ms"] / args.steps,
                "sym_kernel_tflops": tsym["flop"] / (tsym["ms"] / 1e3) / 1e12 if tsym["ms"] else None,
                "bound_pass_ms_per_step": tk["ms"] / args.steps,
                "bound_pass_tflops": tk["flop"] / (tk["ms"] / 1e3) / 1e12 if tk["ms"] else None,
                "pairs_computed_per_step": (tsym["flop"] + tk["flop"]) / args.steps / (2.0 * d)},
        "mst": {"ms": mst_step_ms, "rounds": stats["rounds"], "scanned": stats["scanned"],
                "resolved": stats["resolved"], "skipped": stats["skipped"],
                "scanned_giant": stats["scanned_giant"],
                "components": stats["n_components"],
                "scan_kernel_ms_per_step": ts["ms"] / args.steps,
                "scan_tflops": ts["flop"] / (ts["ms"] / 1e3) / 1e12 if ts["ms"] else None},
        "roofline": {"kernel": dom_name, "bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_MFMA_TFLOPS,
                     "launches": dom["launches"], "avg_launch_ms": dom["ms"] / max(dom["launches"], 1),
                     "traffic": (stored_traffic() if dom_name == "knn_sym_kernel"
                                 and args.workload == "clips_500000x61" else None),
                     "traffic_unit": "bytes per launch that miss the L2 (FETCH_SIZE + WRITE_SIZE, scaled by a "
                                     "copy of known size; served by the MALL or HBM)"},
    }
    # HDBSCAN tail on the host (outside the step): the last step's tree copied to
    # the host and condensed with min_cluster_size 20 (the page's setting)
    t0 = time.perf_counter()
    lo_h, hi_h, w_h = lo.cpu().numpy(), hi.cpu().numpy(), w.cpu().numpy()
    labels = ekh.hdbscan_tail(lo_h, hi_h, w_h, TAIL_MIN_CLUSTER_SIZE)
    tail_ms = 1000.0 * (time.perf_counter() - t0)
    result["hdbscan_tail"] = {
        "ms": tail_ms, "min_cluster_size": TAIL_MIN_CLUSTER_SIZE, "clusters": int(labels.max()) + 1,
        "noise": int((labels < 0).sum()), "where": "host C++ (ekh_hdbscan_tail), device-to-host copy of the tree included",
        "end_to_end_ms": ms_step + tail_ms}
    if not args.no_sections:
        result["clip_sets"] = time_clips(ekh, datagen, oracle_too=not args.no_cpu_baseline)
        g = os.path.join(ROOT, "tests", "golden", args.workload + "_oracle.json")
        if os.path.exists(g) and not args.no_cpu_baseline:
            # the oracle's own run on this workload (make_golden.py), as context for the MST time
            result["mst"]["oracle_stored_seconds"] = json.load(open(g)).get("oracle_seconds")
        result["knn_sections"] = time_sections(ekh, datagen, oracle_too=not args.no_cpu_baseline)
        result["kmeanspp_seeding"] = time_seeding(ekh, datagen, oracle_too=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(X, ms + 1)
        from oracle import hdbscan_tail as otail
        t0 = time.perf_counter()
        otail.hdbscan_tail(lo_h.astype(np.int64), hi_h.astype(np.int64), w_h.astype(np.float64), n,
                           TAIL_MIN_CLUSTER_SIZE)
        result["hdbscan_tail"]["oracle_ms"] = 1000.0 * (time.perf_counter() - t0)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
