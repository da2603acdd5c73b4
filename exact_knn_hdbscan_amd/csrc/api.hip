// Host side of libekh: the C ABI declared in include/ekh.h.
//
// Validation, workspace carving, the chunk / split planner for the dense
// kernels, the Boruvka round loop and the optional kernel timer.  All GPU work
// is enqueued on the caller's stream; nothing here allocates device memory.
#include "ekh.h"
#include "ekh_internal.h"
#include "host_error.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace ekh;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

} // namespace

// Sets the thread-local message for host-only sources of the library.
int ekh::report_error(int code, const char *msg) {
    g_err = msg;
    return code;
}

namespace {

#define EKH_HIP(call)                                                                                                  \
    do {                                                                                                               \
        hipError_t e_ = (call);                                                                                        \
        if (e_ != hipSuccess) return fail(EKH_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));                    \
    } while (0)

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sequential carving of the caller's workspace (also used to size it).
struct Carver {
    char *base;
    size_t used = 0;
    explicit Carver(void *b) : base((char *)b) {}
    template <class T> T *take(size_t count) {
        T *p = base ? (T *)(base + used) : nullptr;
        used += align_up(sizeof(T) * std::max<size_t>(count, 1));
        return p;
    }
};

// ---- kernel timer -----------------------------------------------------------
struct TimerRec {
    int id;
    int dev; // device the events belong to
    hipEvent_t e0, e1;
    double flop;
};
std::mutex g_tmu;
bool g_timer_on = false;
std::vector<TimerRec> g_trecs;
// events of finished records, kept per device for reuse (creating two events
// per timed launch would put host work between the launches)
std::vector<std::pair<int, hipEvent_t>> g_evpool;

// called with g_tmu held
bool take_event(hipEvent_t *e) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    for (size_t k = g_evpool.size(); k-- > 0;) {
        if (g_evpool[k].first == dev) {
            *e = g_evpool[k].second;
            g_evpool.erase(g_evpool.begin() + (std::ptrdiff_t)k);
            return true;
        }
    }
    return hipEventCreate(e) == hipSuccess;
}

struct TimedLaunch {
    TimerRec rec{};
    bool on = false;
    hipStream_t s;
    TimedLaunch(int id, double flop, hipStream_t st) : s(st) {
        std::lock_guard<std::mutex> lk(g_tmu);
        if (!g_timer_on) return;
        rec.id = id;
        rec.flop = flop;
        if (!take_event(&rec.e0)) return;
        if (!take_event(&rec.e1)) {
            hipEventDestroy(rec.e0);
            return;
        }
        hipGetDevice(&rec.dev);
        on = hipEventRecord(rec.e0, s) == hipSuccess;
        if (!on) {
            hipEventDestroy(rec.e0);
            hipEventDestroy(rec.e1);
        }
    }
    // returns the record's position (for timer_set_flop), or -1 when the timer is off
    int64_t done() {
        if (!on) return -1;
        hipEventRecord(rec.e1, s);
        std::lock_guard<std::mutex> lk(g_tmu);
        g_trecs.push_back(rec);
        return (int64_t)g_trecs.size() - 1;
    }
};

// Sets the algorithmic flop of a recorded launch whose work the host learns only
// later (the Boruvka scan: the active points are counted on the device).
void timer_set_flop(int64_t pos, double flop) {
    if (pos < 0) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (pos < (int64_t)g_trecs.size()) g_trecs[(size_t)pos].flop = flop;
}

// ---- kNN planning -----------------------------------------------------------
struct KnnPlan {
    int K, QM, TR, QT;
    int64_t rows;   // rows per chunk
    int64_t tiles;  // database tiles
    int64_t slots;  // workgroups resident at once, per chunk in flight
    int64_t warm;   // warm-up of fresh lists, in tiles
    int64_t part_entries; // split scratch (entries) of the largest chunk
    int conc;       // chunks in flight at once (each on its own stream and scratch)
};

// How one chunk of query tiles is laid out on the grid of one launch: the
// first body_q tiles whole, the rest in `splits` database splits each.
struct ChunkPlan {
    int64_t body_q;
    int splits;
};

constexpr int64_t kMaxLd = int64_t(1) << 48; // keeps f * ld + i within int64 for every f < EKH_MAX_DIM
constexpr int64_t kMinTilesPerSplit = 4;
constexpr int64_t kMaxSplits = 1024;     // a few query tiles against a long database fill the chip
constexpr int64_t kCUs = 256;             // MI355X compute units (fixed, so that a workspace
                                          // query and the run always plan alike)
constexpr int64_t kLdsPerCu = 160 * 1024;
constexpr int64_t kWarmupWork = 12000;    // warm-up of fresh lists, in 32-row tiles x k-steps (measured)
constexpr int kChunkStreams = 2;          // chunks of one kNN call in flight at once (measured: 2 best)

// kNN workgroups resident per CU: one per wave per SIMD that the registers
// allow (four-wave workgroups), fewer if the LDS tile buffers (two, or four
// where the tile loop takes a barrier per two tiles) and their norms do not fit
// that many times (the lists live in registers)
int64_t knn_groups_per_cu(int K, int QM) {
    const int64_t tr = tile_rows(QM), rs = 4 * qm_pad(QM) + 4;
    // tile buffers, their norms, and the slow path's dot products (column blocks x rows per lane)
    const int64_t nbuf = 2 * knn_tiles_per_barrier(QM);
    const int64_t lds = nbuf * tr * rs * 4 + nbuf * tr * 4 + knn_col_blocks(K, QM) * 4 * (tr / 16) * kThreads * 4;
    const int64_t by_lds = kLdsPerCu / lds;
    const int64_t want = knn_waves_per_simd(K, QM);
    return by_lds < want ? (by_lds < 1 ? 1 : by_lds) : want;
}

// Cost of running q query tiles in s database splits: the launch runs in
// rounds of resident workgroups, and every split starts its lists empty (the
// first tiles insert nearly every row, a cost of about kWarmupWork / k-steps
// tiles), so rounds x (tiles per split + that warm-up).
int64_t split_cost(const KnnPlan &p, int64_t q, int64_t s) {
    return (q * s + p.slots - 1) / p.slots * ((p.tiles + s - 1) / s + p.warm);
}

int best_splits(const KnnPlan &p, int64_t q, int64_t *cost) {
    const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(kMaxSplits, p.tiles / kMinTilesPerSplit));
    int64_t best_s = 1, best = -1;
    for (int64_t s = 1; s <= smax; ++s) {
        const int64_t c = split_cost(p, q, s);
        if (best < 0 || c < best) {
            best = c;
            best_s = s;
        }
    }
    *cost = best;
    return (int)best_s;
}

// Layout of a chunk of `rows` query rows.  Either every tile in the same number
// of splits, or (when cheaper) the whole rounds of tiles unsplit and only the
// tiles left over for a last, partly filled round split finely enough to fill
// it: a ragged last round otherwise leaves most of the chip idle while a few
// workgroups stream the whole database.
ChunkPlan plan_chunk(const KnnPlan &p, int64_t rows) {
    const int64_t q = std::max<int64_t>(1, (rows + p.QT - 1) / p.QT);
    int64_t cu;
    ChunkPlan c{0, best_splits(p, q, &cu)};
    const int64_t body = q / p.slots * p.slots;
    if (body > 0 && body < q) {
        int64_t ct;
        const int st = best_splits(p, q - body, &ct);
        if (body / p.slots * (p.tiles + p.warm) + ct < cu) c = ChunkPlan{body, st};
    }
    return c;
}

int64_t chunk_part_entries(const KnnPlan &p, int64_t rows) {
    const ChunkPlan c = plan_chunk(p, rows);
    return c.splits > 1 ? (rows - c.body_q * p.QT) * c.splits * p.K : 0;
}

// Boruvka scan workgroups resident per CU (the two LDS tile buffers with their
// rows' norms, component labels and core distances; the scan keeps one barrier
// per tile: four buffers spill its registers at d <= 64)
int64_t scan_groups_per_cu(int QM) {
    const int64_t tr = tile_rows(QM), rs = 4 * qm_pad(QM) + 4;
    const int64_t lds = 2 * tr * rs * 4 + 2 * 3 * tr * 4;
    const int64_t by_lds = kLdsPerCu / lds;
    const int64_t want = scan_waves_per_simd(QM);
    return by_lds < want ? (by_lds < 1 ? 1 : by_lds) : want;
}

// max_conc: chunks in flight at most (1: everything on the caller's stream)
KnnPlan plan_knn(int64_t n, int64_t m, int d, int k, int64_t max_chunk_dots, int max_conc = kChunkStreams) {
    KnnPlan p{};
    p.K = pick_k(k);
    p.QM = pick_qm(d);
    p.TR = tile_rows(p.QM);
    p.QT = knn_query_tile(p.K, p.QM);
    p.rows = n;
    if (max_chunk_dots > 0 && m > 0) {
        const int64_t r = max_chunk_dots / m / p.QT * p.QT;
        p.rows = std::min<int64_t>(n, std::max<int64_t>(r, p.QT));
    }
    p.tiles = (m + p.TR - 1) / p.TR;
    // Row chunks run kChunkStreams at a time, so each needs to fill only its
    // share of the resident workgroups: fewer database splits, hence fewer
    // list warm-ups per query, than one chunk filling the chip alone.
    const int64_t nchunks = (n + p.rows - 1) / p.rows;
    p.conc = (int)std::max<int64_t>(1, std::min<int64_t>(std::min(kChunkStreams, max_conc), nchunks));
    p.slots = std::max<int64_t>(1, kCUs * knn_groups_per_cu(p.K, p.QM) / p.conc);
    p.warm = kWarmupWork * 32 / (qm_pad(p.QM) * p.TR); // measured at 32-row tiles
    p.part_entries = chunk_part_entries(p, p.rows);
    if (n % p.rows) p.part_entries = std::max(p.part_entries, chunk_part_entries(p, n % p.rows));
    return p;
}


// bt: point-major copy of the database [m, tile_dim(d)], which the tiles and
// the direct-difference kernels read
size_t knn_ws(const KnnPlan &p, int64_t n, int64_t m, bool self, Carver &c, float **nx, float **ny, Entry **part,
              int32_t **idx_scratch = nullptr, int k = 0, float **bt = nullptr, int d = 0) {
    *nx = c.take<float>(n);
    *ny = self ? *nx : c.take<float>(m);
    // one split-list scratch per chunk in flight
    *part = p.part_entries ? c.take<Entry>((size_t)p.part_entries * p.conc) : nullptr;
    if (idx_scratch) *idx_scratch = c.take<int32_t>((size_t)n * k);
    if (bt) *bt = c.take<float>((size_t)m * tile_dim(d));
    return c.used;
}

int check_points(const float *X, int64_t ld, int64_t n, int d, const char *name) {
    if (!X) return fail(EKH_EINVAL, "%s is NULL", name);
    if (n < 1 || n > INT32_MAX) return fail(EKH_EINVAL, "%s: number of points %lld out of range", name, (long long)n);
    if (d < 1 || d > EKH_MAX_DIM) return fail(EKH_EINVAL, "%s: d = %d out of range [1, %d]", name, d, EKH_MAX_DIM);
    if (ld < n) return fail(EKH_EINVAL, "%s: leading dimension %lld < n = %lld", name, (long long)ld, (long long)n);
    if (ld >= kMaxLd) return fail(EKH_EINVAL, "%s: leading dimension %lld >= 2^48", name, (long long)ld);
    return EKH_OK;
}

// Streams for the chunks of one call beyond the caller's own: created on first
// use on each device (non-blocking, default priority) and kept until the
// process ends.  Calls share them; each call orders its work on them through
// its own events, so concurrent calls only queue behind each other.
int chunk_streams(hipStream_t s, hipStream_t (&out)[kChunkStreams - 1]) {
    static std::mutex mu;
    static std::vector<std::vector<hipStream_t>> per_dev;
    int dev = 0, cur = 0;
    EKH_HIP(hipStreamGetDevice(s, &dev));
    EKH_HIP(hipGetDevice(&cur));
    std::lock_guard<std::mutex> lk(mu);
    if ((int)per_dev.size() <= dev) per_dev.resize(dev + 1);
    auto &v = per_dev[dev];
    if (v.empty()) {
        if (cur != dev) EKH_HIP(hipSetDevice(dev));
        std::vector<hipStream_t> made(kChunkStreams - 1, nullptr);
        hipError_t e = hipSuccess;
        for (auto &x : made)
            if (e == hipSuccess) e = hipStreamCreateWithFlags(&x, hipStreamNonBlocking);
        if (cur != dev) hipSetDevice(cur);
        if (e != hipSuccess) {
            for (auto &x : made)
                if (x) hipStreamDestroy(x);
            return fail(EKH_EHIP, "hipStreamCreateWithFlags failed: %s", hipGetErrorString(e));
        }
        v = made;
    }
    for (int i = 0; i < kChunkStreams - 1; ++i) out[i] = v[i];
    return EKH_OK;
}

// Makes `waiter` wait for the work queued so far on `from` (a one-use event).
int stream_wait(hipStream_t waiter, hipStream_t from) {
    hipEvent_t e;
    EKH_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    hipError_t r = hipEventRecord(e, from);
    if (r == hipSuccess) r = hipStreamWaitEvent(waiter, e, 0);
    hipEventDestroy(e); // released once the recorded work completes
    if (r != hipSuccess) return fail(EKH_EHIP, "stream ordering failed: %s", hipGetErrorString(r));
    return EKH_OK;
}

// Runs the dense kNN over all chunks.  out_mode: kOutKnn or kOutCore.
// Chunk c runs on stream c mod p.conc (0 = the caller's) with its own split
// scratch; the other streams start after the norms and the caller's stream
// waits for all of them before anything that reads the outputs.
// core_direct (core mode): the core distances are recomputed by direct
// differences from the final lists (knn_core_kernel), which needs bt.
int run_knn(const KnnPlan &p, const float *X, int64_t ldx, int64_t n, const float *Y, int64_t ldy, int64_t m, int d,
            bool self, int out_mode, int k_out, int min_samples, int32_t *out_idx, float *out_dist, float *out_core,
            float *nx, float *ny, Entry *part, float *bt, hipStream_t s, bool core_direct = false) {
    // norms of both sets and the database's point-major copy, in one launch
    if (!bt) return fail(EKH_EINTERNAL, "no point-major scratch for the database");
    EKH_HIP(launch_prep(X, ldx, n, nx, Y, ldy, m, self ? nullptr : ny, bt, d, tile_dim(d), s));
    hipStream_t cs[kChunkStreams] = {s};
    int forked = 1; // streams in use: the caller's, then those made to wait for it
    // After the fork every exit, an error included, first makes the caller's
    // stream wait for the other streams: the caller may free the workspace and
    // the outputs as soon as its own stream has passed the call's work.
    auto join = [&](int rc) {
        for (int i = 1; i < forked; ++i) {
            const int r = stream_wait(s, cs[i]);
            if (rc == EKH_OK) rc = r;
        }
        return rc;
    };
    if (p.conc > 1) {
        hipStream_t extra[kChunkStreams - 1];
        int rc;
        if ((rc = chunk_streams(s, extra)) != EKH_OK) return rc;
        for (int i = 1; i < p.conc; ++i) {
            cs[i] = extra[i - 1];
            if ((rc = stream_wait(cs[i], s)) != EKH_OK) return join(rc);
            forked = i + 1;
        }
    }
#define EKH_HIP_JOIN(call)                                                                                             \
    do {                                                                                                               \
        hipError_t e_ = (call);                                                                                        \
        if (e_ != hipSuccess) return join(fail(EKH_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)));            \
    } while (0)
    int64_t chunk = 0;
    for (int64_t q0 = 0; q0 < n; q0 += p.rows, ++chunk) {
        const int lane = (int)(chunk % p.conc);
        const hipStream_t cstream = cs[lane];
        KnnArgs a{};
        a.Q = X;
        a.ldq = ldx;
        a.q0 = q0;
        a.nq = std::min<int64_t>(p.rows, n - q0);
        a.nrm_q = nx;
        a.Bt = bt;
        a.dp = tile_dim(d);
        a.m = m;
        a.nrm_b = ny;
        a.d = d;
        a.self = self ? 1 : 0;
        const ChunkPlan cp = plan_chunk(p, a.nq);
        a.body_q = cp.body_q;
        a.splits = cp.splits;
        a.tiles = p.tiles;
        a.k_out = k_out;
        a.min_samples = min_samples;
        a.part = part ? part + (size_t)lane * p.part_entries : nullptr;
        a.out_idx = out_idx;
        a.out_dist = out_dist;
        a.out_core = out_core;
        a.out_mode = out_mode;
        TimedLaunch tl(0, 2.0 * d * (double)a.nq * (double)m, cstream);
        EKH_HIP_JOIN(launch_knn_tile(p.K, p.QM, a, cstream));
        tl.done();
        if (cp.splits > 1) {
            // the split tiles' rows only
            a.q0 += cp.body_q * p.QT;
            a.nq -= cp.body_q * p.QT;
            EKH_HIP_JOIN(launch_knn_merge(p.K, a, cstream));
        }
    }
#undef EKH_HIP_JOIN
    {
        const int rc = join(EKH_OK);
        if (rc != EKH_OK) return rc;
    }
    if (out_mode == kOutKnn) {
        // reported distances, over all rows at once (no rows x m scratch involved)
        KnnArgs a{};
        a.Q = X;
        a.ldq = ldx;
        a.q0 = 0;
        a.nq = n;
        a.m = m;
        a.d = d;
        a.k_out = k_out;
        a.out_idx = out_idx;
        a.out_dist = out_dist;
        a.Bt = bt;
        a.dp = tile_dim(d);
        EKH_HIP(launch_knn_rescore(p.K, a, s));
    } else if (core_direct) {
        KnnArgs a{};
        a.Q = X;
        a.ldq = ldx;
        a.q0 = 0;
        a.nq = n;
        a.m = m;
        a.d = d;
        a.k_out = k_out;
        a.min_samples = min_samples;
        a.out_idx = out_idx;
        a.out_core = out_core;
        a.Bt = bt;
        a.dp = tile_dim(d);
        EKH_HIP(launch_knn_core(p.K, a, s));
    }
    return EKH_OK;
}

// ---- symmetric self-kNN (ekh_core_distances) --------------------------------
// Plan of the symmetric self-kNN: a bound pass of all points against every
// kSymSubset-th point, the symmetric pass over the upper block triangle in
// `splits` pieces per query tile, the merge, and the recomputation of the
// query tiles whose column buffers overflowed.  Taken from kSymMinPoints
// points on at d <= 64 (the kernels' instantiations), unless EKH_CORE_DENSE is
// set in the environment (then every pair is computed from both sides, as in
// ekh_knn).  The workspace query and the call must see the same setting.
struct SymPlan {
    bool on = false;
    int K = 0, QM = 0, TR = 0;
    int QT = 0, GT = 0; // query tile of the symmetric pass; of the dense kernel (the overflow gates' unit)
    int64_t ns = 0, qtiles = 0, gtiles = 0, tiles = 0;
    int splits = 1;
    double pairs = 0; // pairs the symmetric pass computes
    KnnPlan pa{}, pf{};
};

SymPlan plan_sym(int64_t n, int d, int k) {
    SymPlan p;
    p.K = pick_k(k);
    p.QM = pick_qm(d);
    const char *env = getenv("EKH_CORE_DENSE");
    p.on = n >= kSymMinPoints && p.QM <= 16 && p.K > 0 && !(env && env[0] && env[0] != '0');
    if (!p.on) return p;
    p.TR = tile_rows(p.QM);
    p.QT = sym_query_tile(p.K, p.QM);
    p.GT = knn_query_tile(p.K, p.QM);
    p.ns = (n + kSymSubset - 1) / kSymSubset;
    p.qtiles = (n + p.QT - 1) / p.QT;
    p.gtiles = (n + p.GT - 1) / p.GT;
    p.tiles = (n + p.TR - 1) / p.TR;
    // tiles of the triangle; pieces per query tile so that none is longer than
    // half of a resident workgroup's share (the longest run first)
    const int64_t per = p.QT / p.TR;
    int64_t work = 0;
    for (int64_t t = 0; t < p.qtiles; ++t) {
        work += p.tiles - t * per;
        const int64_t q = std::min<int64_t>(p.QT, n - t * p.QT);
        p.pairs += (double)q * (double)(n - t * p.QT);
    }
    // workgroups resident per CU: one per wave per SIMD (the LDS, two tile
    // buffers with the slow path's dot products and the column queue, fits four)
    const int64_t slots = kCUs * sym_waves_per_simd(p.K, p.QM);
    while (p.splits < kSymMaxSplits && (p.tiles + p.splits - 1) / p.splits * 2 * slots > work) ++p.splits;
    p.pa = plan_knn(n, p.ns, d, k, 0, 1);
    p.pf = plan_knn(n, n, d, k, 0, 1);
    return p;
}

struct SymWs {
    float *nx, *bt, *bs, *nrm_s, *tau, *theta;
    int32_t *idx;
    Entry *part_a, *part_b, *part_f, *colbuf;
    uint32_t *colcnt, *gate;
};

size_t sym_ws(const SymPlan &p, int64_t n, int d, int k, Carver &c, SymWs &w) {
    const int dp = tile_dim(d);
    w.nx = c.take<float>(n);
    w.bt = c.take<float>((size_t)n * dp);
    w.idx = c.take<int32_t>((size_t)n * k);
    w.bs = c.take<float>((size_t)p.ns * dp);
    w.nrm_s = c.take<float>(p.ns);
    w.part_a = p.pa.part_entries ? c.take<Entry>((size_t)p.pa.part_entries) : nullptr;
    w.tau = c.take<float>(n);
    w.theta = c.take<float>(n);
    w.part_b = c.take<Entry>((size_t)p.splits * n * p.K);
    w.colbuf = c.take<Entry>((size_t)n * kSymColCap);
    w.colcnt = c.take<uint32_t>(n);
    w.gate = c.take<uint32_t>(p.gtiles);
    w.part_f = p.pf.part_entries ? c.take<Entry>((size_t)p.pf.part_entries) : nullptr;
    return c.used;
}

// One pass of a kNN plan with a single chunk (no row chunking), on stream s:
// the tile launch and, for split tiles, their merge.  flop: the launch's
// algorithmic flop for the timer (0 where the device decides the work: the
// launch's time then counts with no flop).
int run_single_chunk(const KnnPlan &p, KnnArgs a, double flop, hipStream_t s) {
    const ChunkPlan cp = plan_chunk(p, a.nq);
    a.body_q = cp.body_q;
    a.splits = cp.splits;
    a.tiles = p.tiles;
    TimedLaunch tl(0, flop, s);
    EKH_HIP(launch_knn_tile(p.K, p.QM, a, s));
    tl.done();
    if (cp.splits > 1) {
        a.q0 += cp.body_q * p.QT;
        a.nq -= cp.body_q * p.QT;
        EKH_HIP(launch_knn_merge(p.K, a, s));
    }
    return EKH_OK;
}

int run_core_sym(const SymPlan &p, const float *X, int64_t ldx, int64_t n, int d, int ms, int32_t *out_idx,
                 float *out_d2, float *out_core, const SymWs &w, hipStream_t s) {
    const int k = ms + 1, dp = tile_dim(d);
    int rc;
    // norms and the point-major copy, then the subset's rows
    EKH_HIP(launch_prep(X, ldx, n, w.nx, X, ldx, n, nullptr, w.bt, d, dp, s));
    EKH_HIP(launch_subset_gather(w.bt, w.nx, n, dp, kSymSubset, w.bs, w.nrm_s, s));
    KnnArgs a{};
    a.Q = X;
    a.ldq = ldx;
    a.q0 = 0;
    a.nq = n;
    a.nrm_q = w.nx;
    a.d = d;
    a.dp = dp;
    a.k_out = k;
    a.min_samples = ms;
    // bound pass: tau = D2 of each point's k-th neighbour among the subset
    {
        KnnArgs b = a;
        b.Bt = w.bs;
        b.m = p.ns;
        b.nrm_b = w.nrm_s;
        b.part = w.part_a;
        b.out_mode = kOutBound;
        b.out_core = w.tau;
        if ((rc = run_single_chunk(p.pa, b, 2.0 * d * (double)n * (double)p.ns, s)) != EKH_OK) return rc;
    }
    EKH_HIP(launch_sym_setup(w.tau, w.nx, n, w.theta, w.colcnt, w.gate, p.gtiles, s));
    // symmetric pass over the upper block triangle
    a.Bt = w.bt;
    a.m = n;
    a.nrm_b = w.nx;
    a.self = 1;
    a.tiles = p.tiles;
    a.splits = p.splits;
    a.part = w.part_b;
    a.tau = w.tau;
    a.theta = w.theta;
    a.colbuf = w.colbuf;
    a.colcnt = w.colcnt;
    a.colcap = kSymColCap;
    {
        TimedLaunch tl(2, 2.0 * d * p.pairs, s);
        EKH_HIP(launch_knn_sym(p.K, p.QM, a, s));
        tl.done();
    }
    // final lists: the row side's pieces with the column side's candidates
    a.out_mode = kOutCore;
    a.out_idx = out_idx;
    a.out_dist = out_d2;
    a.out_core = out_core;
    a.gate_w = w.gate;
    a.gate_rows = p.GT;
    EKH_HIP(launch_sym_merge(p.K, a, s));
    // the query tiles with an overflowed buffer, recomputed from both sides
    {
        KnnArgs f = a;
        f.tau = nullptr;
        f.theta = nullptr;
        f.colbuf = nullptr;
        f.colcnt = nullptr;
        f.gate_w = nullptr;
        f.gate = w.gate;
        f.part = w.part_f;
        if ((rc = run_single_chunk(p.pf, f, 0.0, s)) != EKH_OK) return rc;
    }
    // core distances by direct differences from the final lists
    KnnArgs c{};
    c.Q = X;
    c.ldq = ldx;
    c.q0 = 0;
    c.nq = n;
    c.m = n;
    c.d = d;
    c.k_out = k;
    c.min_samples = ms;
    c.out_idx = out_idx;
    c.out_core = out_core;
    c.Bt = w.bt;
    c.dp = dp;
    EKH_HIP(launch_knn_core(p.K, c, s));
    return EKH_OK;
}

// ---- MST workspace ----------------------------------------------------------
struct MstWs {
    float *nrm;
    int32_t *comp, *parent, *act;
    uint8_t *resolved;
    float *lbound;
    uint64_t *best, *cmin1, *cc;
    uint32_t *cmin2, *compW;
    int32_t *e_lo, *e_hi;
    float *e_w;
    uint32_t *sa, *sb, *sc, *sd;
    uint64_t *s64a, *s64b;
    void *sort_tmp;
    size_t sort_tmp_bytes;
    BvCounters *ctr;
    int32_t *nbr_idx;
    float *nbr_d2;
    float *knn_nx;
    Entry *knn_part;
    float *xs; // points outside the largest component, point-major [<= n / 2, tile_dim(d)]
    float *pm; // point-major copy [n, tile_dim(d)]: the scans' database and the reported edge weights
};

size_t carve_mst(Carver &c, int64_t n, int d, int ms, bool with_nb, MstWs &w) {
    w.nrm = c.take<float>(n);
    w.comp = c.take<int32_t>(n);
    w.cc = c.take<uint64_t>(n);
    w.parent = c.take<int32_t>(n);
    w.act = c.take<int32_t>(n);
    w.resolved = c.take<uint8_t>(n);
    w.lbound = c.take<float>(n);
    w.best = c.take<uint64_t>(n);
    w.cmin1 = c.take<uint64_t>(n);
    w.cmin2 = c.take<uint32_t>(n);
    w.compW = c.take<uint32_t>(n);
    w.e_lo = c.take<int32_t>(n);
    w.e_hi = c.take<int32_t>(n);
    w.e_w = c.take<float>(n);
    w.sa = c.take<uint32_t>(n);
    w.sb = c.take<uint32_t>(n);
    w.sc = c.take<uint32_t>(n);
    w.sd = c.take<uint32_t>(n);
    w.s64a = c.take<uint64_t>(n);
    w.s64b = c.take<uint64_t>(n);
    w.sort_tmp_bytes = edge_sort_temp_bytes(n - 1);
    w.sort_tmp = c.take<char>(w.sort_tmp_bytes);
    w.ctr = c.take<BvCounters>(1);
    // the largest component's complement (used when it holds >= n / 2 points):
    // its points' features here; orig, labels, sizes and the second active list
    // in the edge sort's u32 scratch (sb, sc, sd, sa), norms and core distances
    // in s64a -- all idle until the final sort
    w.xs = c.take<float>((size_t)tile_dim(d) * (size_t)(n / 2 + 1));
    w.pm = c.take<float>((size_t)n * (size_t)tile_dim(d));
    w.nbr_idx = nullptr;
    w.nbr_d2 = nullptr;
    w.knn_nx = nullptr;
    w.knn_part = nullptr;
    if (!with_nb) {
        const int K = ms + 1;
        w.nbr_idx = c.take<int32_t>((size_t)n * K);
        w.nbr_d2 = c.take<float>((size_t)n * K);
        const KnnPlan p = plan_knn(n, n, d, K, 0);
        float *ny; // knn_ws also carves norms, unused here: the call writes w.nrm
        knn_ws(p, n, n, true, c, &w.knn_nx, &ny, &w.knn_part);
    }
    return c.used;
}

int ceil_log2(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}

} // namespace

// ---- scratch of ekh_knn_noalloc -----------------------------------------------
// One array per GPU (each device holds its own copy, at its own address), kept
// until the process ends.  In host code `scratch` names a host-side stand-in,
// never the device memory: host code uses only the address that
// hipGetSymbolAddress returns for the device, taken once per device with that
// device current, and passes that to the kernels.
static __device__ __align__(256) unsigned char scratch[EKH_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::vector<void *> g_scratch_dev; // device address of `scratch`, per device

// Device address of `scratch` on the device of stream s.
int noalloc_scratch(hipStream_t s, void **out) {
    int cur = 0, dev = 0;
    EKH_HIP(hipGetDevice(&cur));
    if (s) EKH_HIP(hipStreamGetDevice(s, &dev));
    else dev = cur;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_dev.size() <= dev) g_scratch_dev.resize((size_t)dev + 1, nullptr);
    if (!g_scratch_dev[(size_t)dev]) {
        if (cur != dev) EKH_HIP(hipSetDevice(dev));
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return fail(EKH_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_dev[(size_t)dev] = p;
    }
    *out = g_scratch_dev[(size_t)dev];
    return EKH_OK;
}

} // namespace

extern "C" {

int ekh_version(void) { return 100; }

const char *ekh_last_error(void) { return g_err.c_str(); }

size_t ekh_knn_workspace_bytes(int64_t n, int64_t m, int32_t d, int32_t k, int64_t max_chunk_dots) {
    if (n < 1 || m < 1 || d < 1 || d > EKH_MAX_DIM || k < 1 || k > EKH_MAX_K) return 0;
    const KnnPlan p = plan_knn(n, m, d, k, max_chunk_dots);
    Carver c(nullptr);
    float *nx, *ny;
    Entry *part;
    int32_t *idx;
    float *bt;
    return knn_ws(p, n, m, false, c, &nx, &ny, &part, &idx, k, &bt, d);
}

int ekh_knn_plan(int64_t n, int64_t m, int32_t d, int32_t k, int64_t max_chunk_dots, int64_t out[8]) {
    if (!out) return fail(EKH_EINVAL, "out is NULL");
    if (n < 1 || n > INT32_MAX || m < 1 || m > INT32_MAX || d < 1 || d > EKH_MAX_DIM || k < 1 || k > EKH_MAX_K ||
        k > m)
        return fail(EKH_EINVAL, "sizes out of range (n %lld, m %lld, d %d, k %d)", (long long)n, (long long)m, d, k);
    const KnnPlan p = plan_knn(n, m, d, k, max_chunk_dots);
    const ChunkPlan first = plan_chunk(p, std::min(p.rows, n));
    const ChunkPlan last = plan_chunk(p, n % p.rows ? n % p.rows : p.rows);
    out[0] = p.rows;
    out[1] = p.QT;
    out[2] = first.body_q;
    out[3] = first.splits;
    out[4] = p.slots;
    out[5] = last.body_q;
    out[6] = last.splits;
    out[7] = p.conc;
    return EKH_OK;
}

int ekh_knn(const float *X, int64_t ldx, int64_t n, const float *Y, int64_t ldy, int64_t m, int32_t d, int32_t k,
            int32_t *out_idx, float *out_dist, int64_t max_chunk_dots, void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_points(X, ldx, n, d, "X")) != EKH_OK) return rc;
    if ((rc = check_points(Y, ldy, m, d, "Y")) != EKH_OK) return rc;
    if (k < 1 || k > EKH_MAX_K || k > m) return fail(EKH_EINVAL, "k = %d out of range [1, min(m, %d)]", k, EKH_MAX_K);
    if (max_chunk_dots < 0) return fail(EKH_EINVAL, "max_chunk_dots < 0");
    if (!out_idx && !out_dist) return fail(EKH_EINVAL, "no output requested");
    if (!ws) return fail(EKH_EINVAL, "workspace is NULL");
    const size_t need = ekh_knn_workspace_bytes(n, m, d, k, max_chunk_dots);
    if (ws_bytes < need) return fail(EKH_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    const bool self = (X == Y) && (ldx == ldy) && (n == m);
    const KnnPlan p = plan_knn(n, m, d, k, max_chunk_dots);
    Carver c(ws);
    float *nx, *ny;
    Entry *part;
    int32_t *idx_scratch;
    float *bt;
    knn_ws(p, n, m, false, c, &nx, &ny, &part, &idx_scratch, k, &bt, d);
    if (self) ny = nx;
    return run_knn(p, X, ldx, n, Y, ldy, m, d, self, kOutKnn, k, 0, out_idx ? out_idx : idx_scratch, out_dist,
                   nullptr, nx, ny, part, bt, (hipStream_t)stream);
}

size_t ekh_core_workspace_bytes(int64_t n, int32_t d, int32_t min_samples) {
    if (n < 1 || d < 1 || d > EKH_MAX_DIM || min_samples < 1 || min_samples + 1 > EKH_MAX_K) return 0;
    const SymPlan sp = plan_sym(n, d, min_samples + 1);
    if (sp.on) {
        Carver c(nullptr);
        SymWs w;
        return sym_ws(sp, n, d, min_samples + 1, c, w);
    }
    const KnnPlan p = plan_knn(n, n, d, min_samples + 1, 0);
    Carver c(nullptr);
    float *nx, *ny, *bt;
    Entry *part;
    int32_t *idx;
    return knn_ws(p, n, n, true, c, &nx, &ny, &part, &idx, min_samples + 1, &bt, d);
}

int ekh_core_distances(const float *X, int64_t ldx, int64_t n, int32_t d, int32_t min_samples, float *out_core,
                       int32_t *out_nbr_idx, float *out_nbr_d2, void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_points(X, ldx, n, d, "X")) != EKH_OK) return rc;
    if (min_samples < 1 || min_samples + 1 > EKH_MAX_K || min_samples >= n)
        return fail(EKH_EINVAL, "min_samples = %d out of range [1, min(n - 1, %d)]", min_samples, EKH_MAX_K - 1);
    if (!out_core) return fail(EKH_EINVAL, "out_core is NULL");
    if ((out_nbr_idx == nullptr) != (out_nbr_d2 == nullptr))
        return fail(EKH_EINVAL, "out_nbr_idx and out_nbr_d2 must both be NULL or both be set");
    if (!ws) return fail(EKH_EINVAL, "workspace is NULL");
    const size_t need = ekh_core_workspace_bytes(n, d, min_samples);
    if (ws_bytes < need) return fail(EKH_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    const int K = min_samples + 1;
    const SymPlan sp = plan_sym(n, d, K);
    if (sp.on) {
        Carver c(ws);
        SymWs w;
        sym_ws(sp, n, d, K, c, w);
        return run_core_sym(sp, X, ldx, n, d, min_samples, out_nbr_idx ? out_nbr_idx : w.idx, out_nbr_d2, out_core, w,
                            (hipStream_t)stream);
    }
    const KnnPlan p = plan_knn(n, n, d, K, 0);
    Carver c(ws);
    float *nx, *ny, *bt;
    Entry *part;
    int32_t *idx_scratch;
    knn_ws(p, n, n, true, c, &nx, &ny, &part, &idx_scratch, K, &bt, d);
    return run_knn(p, X, ldx, n, X, ldx, n, d, true, kOutCore, K, min_samples, out_nbr_idx ? out_nbr_idx : idx_scratch,
                   out_nbr_d2, out_core, nx, nx, part, bt, (hipStream_t)stream, true);
}

size_t ekh_mst_workspace_bytes(int64_t n, int32_t d, int32_t min_samples, int with_neighbours) {
    if (n < 1 || d < 1 || d > EKH_MAX_DIM || min_samples < 1 || min_samples + 1 > EKH_MAX_K) return 0;
    Carver c(nullptr);
    MstWs w;
    return carve_mst(c, n, d, min_samples, with_neighbours != 0, w);
}

int ekh_mst_boruvka(const float *X, int64_t ldx, int64_t n, int32_t d, const float *core, int32_t min_samples,
                    const int32_t *nbr_idx, const float *nbr_d2, uint32_t flags, int32_t *out_lo, int32_t *out_hi,
                    float *out_w, ekh_mst_stats *stats, void *ws, size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_points(X, ldx, n, d, "X")) != EKH_OK) return rc;
    if (!core) return fail(EKH_EINVAL, "core is NULL");
    if (min_samples < 1 || min_samples + 1 > EKH_MAX_K || (n >= 2 && min_samples >= n))
        return fail(EKH_EINVAL, "min_samples = %d out of range [1, min(n - 1, %d)]", min_samples, EKH_MAX_K - 1);
    if ((nbr_idx == nullptr) != (nbr_d2 == nullptr))
        return fail(EKH_EINVAL, "nbr_idx and nbr_d2 must both be NULL or both be set");
    if (flags & ~(EKH_MST_NO_NEIGHBOUR_EDGES | EKH_MST_NO_COMPONENT_BOUND | EKH_MST_FULL_SCANS))
        return fail(EKH_EINVAL, "unknown flags");
    if (n >= 2 && (!out_lo || !out_hi || !out_w)) return fail(EKH_EINVAL, "edge outputs are NULL");
    if (!ws) return fail(EKH_EINVAL, "workspace is NULL");
    const bool with_nb = nbr_idx != nullptr;
    const size_t need = ekh_mst_workspace_bytes(n, d, min_samples, with_nb ? 1 : 0);
    if (ws_bytes < need) return fail(EKH_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    if (stats) std::memset(stats, 0, sizeof *stats);
    if (n == 1) return EKH_OK;

    hipStream_t s = (hipStream_t)stream;
    Carver c(ws);
    MstWs w;
    carve_mst(c, n, d, min_samples, with_nb, w);
    const int K = min_samples + 1;

    if (!with_nb) {
        // the self-kNN rows (K = min_samples + 1) the shortcuts read; the call
        // also leaves the norms and the point-major copy of X
        const KnnPlan p = plan_knn(n, n, d, K, 0);
        float *scratch_core = (float *)w.sa; // core as computed here is not used: the caller's core rules
        if ((rc = run_knn(p, X, ldx, n, X, ldx, n, d, true, kOutCore, K, min_samples, w.nbr_idx, w.nbr_d2,
                          scratch_core, w.nrm, w.nrm, w.knn_part, w.pm, s)) != EKH_OK)
            return rc;
        nbr_idx = w.nbr_idx;
        nbr_d2 = w.nbr_d2;
    } else {
        // norms and the point-major copy of X, in one launch
        EKH_HIP(launch_prep(X, ldx, n, w.nrm, X, ldx, n, nullptr, w.pm, d, tile_dim(d), s));
    }

    BvState st{};
    st.n = n;
    st.K = K;
    st.nbr_idx = nbr_idx;
    st.nbr_d2 = nbr_d2;
    st.core = core;
    st.comp = w.comp;
    st.cc = w.cc;
    st.parent = w.parent;
    st.act = w.act;
    st.resolved = w.resolved;
    st.lbound = w.lbound;
    st.best = w.best;
    st.cmin1 = w.cmin1;
    st.cmin2 = w.cmin2;
    st.compW = w.compW;
    st.csize = w.sd;
    st.act_g = reinterpret_cast<int32_t *>(w.sa);
    st.e_lo = w.e_lo;
    st.e_hi = w.e_hi;
    st.e_w = w.e_w;
    st.ctr = w.ctr;

    const int use_nb = (flags & EKH_MST_NO_NEIGHBOUR_EDGES) ? 0 : 1;
    const int use_bound = (flags & EKH_MST_NO_COMPONENT_BOUND) ? 0 : 1;
    const bool giant_scans = !(flags & EKH_MST_FULL_SCANS);
    const int QM = pick_qm(d);
    const int TR = tile_rows(QM);
    const int64_t tiles = (n + TR - 1) / TR;
    const int64_t scan_grid = kCUs * scan_groups_per_cu(QM); // one round of resident workgroups
    const int cap = std::max(1, ceil_log2(n));

    ScanArgs sa{};
    sa.X = X;
    sa.ldx = ldx;
    sa.n = n;
    sa.nrm = w.nrm;
    sa.core = core;
    sa.comp = w.comp;
    sa.compW = w.compW;
    sa.best = w.best;
    sa.d = d;

    // One host read-back per round, after the merge: the scans size their work
    // from the device-side active counts, and the largest component of the next
    // round (size << 32 | label) is counted before the read-back.
    EKH_HIP(bv_init(st, s));
    int64_t ncomp = n;
    int round = 0;
    BvCounters h{};
    while (ncomp > 1) {
        if (round >= cap)
            return fail(EKH_EINTERNAL, "Boruvka did not finish in %d rounds (%lld components left)", cap,
                        (long long)ncomp);
        const auto t0 = std::chrono::steady_clock::now();
        // the largest component, when it holds >= n / 2 points: its active points
        // are scanned only against the points outside it (a cheapest edge leaves
        // the component)
        const int64_t sg = (int64_t)(h.giant >> 32), ns = n - sg;
        const int32_t g = (int32_t)(uint32_t)h.giant;
        const int split_giant = round > 0 && giant_scans && sg * 2 >= n && ns >= 1 ? 1 : 0;
        EKH_HIP(bv_reset_counters(st, s));
        EKH_HIP(bv_candidates(st, use_nb, use_bound, s));
        EKH_HIP(bv_select_active(st, use_bound, split_giant, s));
        sa.Xb = w.pm;
        sa.dp = tile_dim(d);
        sa.nb = n;
        sa.nrm_b = w.nrm;
        sa.core_b = core;
        sa.comp_b = w.comp;
        sa.orig = nullptr;
        sa.act = w.act;
        sa.nact = &w.ctr->n_active;
        sa.tiles = tiles;
        TimedLaunch tl(1, 0.0, s);
        EKH_HIP(launch_scan_tile(QM, sa, scan_grid, s));
        const int64_t t_main = tl.done();
        int64_t t_giant = -1;
        if (split_giant) {
            int32_t *orig = reinterpret_cast<int32_t *>(w.sb);
            int32_t *comp_s = reinterpret_cast<int32_t *>(w.sc);
            float *nrm_s = reinterpret_cast<float *>(w.s64a), *core_s = nrm_s + (n / 2 + 1);
            // both do nothing when no active point of the component was listed
            EKH_HIP(bv_complement(st, g, orig, s));
            EKH_HIP(bv_gather_points(w.pm, tile_dim(d), orig, ns, w.nrm, core, w.comp, w.xs, nrm_s, core_s, comp_s,
                                     &w.ctr->n_comp_g, &w.ctr->n_active_g, s));
            sa.Xb = w.xs;
            sa.nb = ns;
            sa.nrm_b = nrm_s;
            sa.core_b = core_s;
            sa.comp_b = comp_s;
            sa.orig = orig;
            sa.act = st.act_g;
            sa.nact = &w.ctr->n_active_g;
            sa.tiles = (ns + TR - 1) / TR;
            TimedLaunch tg(1, 0.0, s);
            EKH_HIP(launch_scan_tile(QM, sa, scan_grid, s));
            t_giant = tg.done();
        }
        EKH_HIP(bv_component_min(st, s));
        EKH_HIP(bv_select_edges(st, s));
        const int jumps = ceil_log2(ncomp) + 1;
        for (int j = 0; j < jumps; ++j) EKH_HIP(bv_jump(st, s));
        EKH_HIP(bv_relabel(st, s));
        if (giant_scans) EKH_HIP(bv_giant(st, s)); // for the next round
        EKH_HIP(hipMemcpyAsync(&h, w.ctr, sizeof h, hipMemcpyDeviceToHost, s));
        EKH_HIP(hipStreamSynchronize(s));
        const int64_t nact = h.n_active, nact_g = split_giant ? h.n_active_g : 0;
        timer_set_flop(t_main, 2.0 * d * (double)nact * (double)n);
        timer_set_flop(t_giant, 2.0 * d * (double)nact_g * (double)ns);
        if (h.n_missing) return fail(EKH_EINTERNAL, "round %d: %u components found no outgoing edge", round, h.n_missing);
        if (split_giant && nact_g > 0 && (int64_t)h.n_comp_g != ns)
            return fail(EKH_EINTERNAL, "round %d: %u points outside the largest component, expected %lld", round,
                        h.n_comp_g, (long long)ns);
        const int64_t before = ncomp;
        ncomp = h.n_roots;
        if (ncomp >= before || ncomp < 1)
            return fail(EKH_EINTERNAL, "round %d: components %lld -> %lld", round, (long long)before, (long long)ncomp);
        if (stats && round < EKH_MAX_ROUNDS) {
            stats->n_components[round] = (int32_t)ncomp;
            stats->resolved[round] = h.n_resolved;
            stats->skipped[round] = h.n_skipped;
            stats->scanned[round] = nact + nact_g;
            stats->scanned_giant[round] = nact_g;
            stats->edges_added[round] = before - ncomp;
            stats->round_ms[round] =
                std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
        }
        ++round;
    }
    if (stats) stats->rounds = round;
    if ((int64_t)h.n_edges != n - 1)
        return fail(EKH_EINTERNAL, "tree has %u edges, expected %lld", h.n_edges, (long long)(n - 1));
    // each edge's reported weight by direct differences, then the (w, lo, hi) order
    EKH_HIP(bv_edge_weights(w.pm, tile_dim(d), core, w.e_lo, w.e_hi, n - 1, n, w.e_w, s));
    EKH_HIP(edge_sort(w.e_lo, w.e_hi, w.e_w, n - 1, w.sort_tmp, w.sort_tmp_bytes, w.sa, w.sb, w.sc, w.sd, w.s64a,
                      w.s64b, out_lo, out_hi, out_w, s));
    return EKH_OK;
}

size_t ekh_knn_noalloc_bytes(int64_t n, int64_t m, int32_t d, int32_t k, int64_t max_chunk_dots) {
    if (n < 1 || m < 1 || d < 1 || d > EKH_MAX_DIM || k < 1 || k > EKH_MAX_K) return 0;
    const KnnPlan p = plan_knn(n, m, d, k, max_chunk_dots, 1);
    Carver c(nullptr);
    float *nx, *ny, *bt;
    Entry *part;
    int32_t *idx;
    return knn_ws(p, n, m, false, c, &nx, &ny, &part, &idx, k, &bt, d);
}

int ekh_knn_noalloc(const float *X, int64_t ldx, int64_t n, const float *Y, int64_t ldy, int64_t m, int32_t d,
                    int32_t k, int32_t *out_idx, float *out_dist, int64_t max_chunk_dots, void *stream) {
    int rc;
    if ((rc = check_points(X, ldx, n, d, "X")) != EKH_OK) return rc;
    if ((rc = check_points(Y, ldy, m, d, "Y")) != EKH_OK) return rc;
    if (k < 1 || k > EKH_MAX_K || k > m) return fail(EKH_EINVAL, "k = %d out of range [1, min(m, %d)]", k, EKH_MAX_K);
    if (max_chunk_dots < 0) return fail(EKH_EINVAL, "max_chunk_dots < 0");
    if (!out_idx && !out_dist) return fail(EKH_EINVAL, "no output requested");
    const size_t need = ekh_knn_noalloc_bytes(n, m, d, k, max_chunk_dots);
    if (need > (size_t)EKH_NOALLOC_SCRATCH_BYTES)
        return fail(EKH_EWORKSPACE, "ekh_knn_noalloc needs %zu bytes of scratch for these sizes; its static scratch holds %zu",
                    need, (size_t)EKH_NOALLOC_SCRATCH_BYTES);
    hipStream_t s = (hipStream_t)stream;
    void *ws = nullptr;
    if ((rc = noalloc_scratch(s, &ws)) != EKH_OK) return rc;
    const bool self = (X == Y) && (ldx == ldy) && (n == m);
    const KnnPlan p = plan_knn(n, m, d, k, max_chunk_dots, 1); // every chunk on the caller's stream
    Carver c(ws);
    float *nx, *ny, *bt;
    Entry *part;
    int32_t *idx_scratch;
    knn_ws(p, n, m, false, c, &nx, &ny, &part, &idx_scratch, k, &bt, d);
    if (self) ny = nx;
    return run_knn(p, X, ldx, n, Y, ldy, m, d, self, kOutKnn, k, 0, out_idx ? out_idx : idx_scratch, out_dist,
                   nullptr, nx, ny, part, bt, s);
}

int ekh_timer_enable(int on) {
    std::lock_guard<std::mutex> lk(g_tmu);
    // the records' events go back to the pool (the caller reads the timer after
    // synchronising, so their work has completed)
    for (auto &r : g_trecs) {
        g_evpool.emplace_back(r.dev, r.e0);
        g_evpool.emplace_back(r.dev, r.e1);
    }
    g_trecs.clear();
    g_timer_on = on != 0;
    return EKH_OK;
}

int ekh_timer_read(int kernel_id, int64_t *launches, double *total_ms, double *algo_flop) {
    if (kernel_id < 0 || kernel_id > 2) return fail(EKH_EINVAL, "unknown kernel id %d", kernel_id);
    std::lock_guard<std::mutex> lk(g_tmu);
    int64_t cnt = 0;
    double ms = 0.0, fl = 0.0;
    for (auto &r : g_trecs) {
        if (r.id != kernel_id) continue;
        if (hipEventSynchronize(r.e1) != hipSuccess) return fail(EKH_EHIP, "hipEventSynchronize failed");
        float t = 0.f;
        if (hipEventElapsedTime(&t, r.e0, r.e1) != hipSuccess) return fail(EKH_EHIP, "hipEventElapsedTime failed");
        ++cnt;
        ms += t;
        fl += r.flop;
    }
    if (launches) *launches = cnt;
    if (total_ms) *total_ms = ms;
    if (algo_flop) *algo_flop = fl;
    return EKH_OK;
}

} // extern "C"
