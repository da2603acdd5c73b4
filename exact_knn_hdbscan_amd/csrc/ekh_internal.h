// Internal declarations of libekh (not part of the C ABI).
//
// The two dense kernels (kNN tile, Boruvka scan tile) share one MFMA tile loop:
// the "query" points of a workgroup are held in registers as the B operand of
// v_mfma_f32_16x16x4_f32, database points stream through LDS as the A
// operand, and each 16 x 16 result block is consumed in registers by an
// epilogue (top-K insertion, or cheapest-edge search).  Squared distances are
// (|q|^2 + |b|^2) - 2 q.b, as on the clustering page ("k-nearest neighbours
// are a matrix product").
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ekh {

// ---- tile geometry -------------------------------------------------------
constexpr int kWaves = 4;             // waves per workgroup (two workgroups per CU)
constexpr int kThreads = kWaves * 64; // 256 threads

// QM = k-steps of the contraction (one feature per lane group each, four per
// k-step), 2 * ceil(d / 8): the tile kernels are instantiated for every even
// QM (2, 4, ..., 64), so the k-loop is always fully unrolled with no runtime
// guard.  Lane group g supplies features g * QM .. g * QM + QM - 1; in a
// point-major row each group's features fill a segment of qm_pad(QM) (QM
// rounded up to 4) positions, zero past QM, so a lane reads four k-steps of
// its operand with one aligned 16-byte read.
// CB = 16-column query blocks per wave; TR = database rows per LDS tile.
constexpr int kMaxQM = 64;
template <int QM> struct TileGeo {
    // d > 224: 16-row tiles keep the prefetch registers and the LDS tile small
    // enough for two workgroups per CU without spills
    static constexpr int TR = QM > 56 ? 16 : 32;
};

// instantiated list lengths; a request for k uses the smallest K >= k
constexpr int kNumK = 7;
constexpr int kKList[kNumK] = {2, 4, 8, 10, 11, 16, 32};
inline int pick_k(int k) {
    for (int i = 0; i < kNumK; ++i)
        if (k <= kKList[i]) return kKList[i];
    return -1;
}
// k-steps run for dimension d (identical in every kernel, which keeps D2
// bitwise the same everywhere), and the positions of one lane group's segment
__host__ __device__ constexpr int pick_qm(int d) { return 2 * ((d + 7) / 8); }
__host__ __device__ constexpr int qm_pad(int qm) { return (qm + 3) & ~3; }
inline int tile_rows(int qm) { return qm > 56 ? 16 : 32; }
// kNN tile kernel occupancy: three waves per SIMD where the registers fit
// without spills (d <= 64 and K <= 16; d <= 128 and K <= 11), two otherwise
constexpr int knn_waves_per_simd(int K, int QM) { return (QM <= 16 && K <= 16) || (QM <= 32 && K <= 11) ? 3 : 2; }
// Boruvka scan kernel occupancy: four waves per SIMD for d <= 64 (one column
// block per wave: 125 VGPRs), three for d <= 128, two otherwise
constexpr int scan_waves_per_simd(int QM) { return QM <= 16 ? 4 : QM <= 32 ? 3 : 2; }
// kNN tiles per barrier of the tile loop: two (four LDS tile buffers) where
// they fit three workgroups per CU, d <= 64
constexpr int knn_tiles_per_barrier(int QM) { return QM <= 16 ? 2 : 1; }
// 16-column query blocks per wave: two when the registers allow it
constexpr int knn_col_blocks(int K, int QM) { return (K > 11 || QM > 16) ? 1 : 2; }
constexpr int scan_col_blocks(int) { return 1; }
inline int knn_query_tile(int K, int QM) { return kWaves * 16 * knn_col_blocks(K, QM); }
// symmetric pass: one 16-column query block per wave and no LDS beyond the tile
// loop's, so that the kernel runs five waves per SIMD up to K = 11 (96 VGPRs),
// four at K = 16 (128)
constexpr int sym_col_blocks(int, int) { return 1; }
constexpr int sym_waves_per_simd(int K, int QM) { return K <= 11 ? 5 : K <= 16 ? 4 : knn_waves_per_simd(K, QM); }
inline int sym_query_tile(int K, int QM) { return kWaves * 16 * sym_col_blocks(K, QM); }
inline int scan_query_tile(int QM) { return kWaves * 16 * scan_col_blocks(QM); }
// row stride (floats) of the point-major copies the tiles read: four segments
// of qm_pad(QM) positions (16 * ceil(d / 16) floats); position g * qm_pad(QM) + s
// holds feature g * QM + s for s < QM and g * QM + s < d, every other position
// zero
__host__ __device__ constexpr int tile_dim(int d) { return 4 * qm_pad(pick_qm(d)); }
// feature at position p of a point-major row (-1: a zero position)
__host__ __device__ constexpr int pm_feature(int p, int qm, int d) {
    const int qp = qm_pad(qm), s = p % qp, f = (p / qp) * qm + s;
    return s < qm && f < d ? f : -1;
}

// X(QM) for every instantiated QM (the even numbers up to kMaxQM), e.g. the
// cases of a switch on a runtime QM.
#define EKH_FOR_EACH_QM(X)                                                                                             \
    X(2) X(4) X(6) X(8) X(10) X(12) X(14) X(16) X(18) X(20) X(22) X(24) X(26) X(28) X(30) X(32) X(34) X(36) X(38)     \
        X(40) X(42) X(44) X(46) X(48) X(50) X(52) X(54) X(56) X(58) X(60) X(62) X(64)

// Correctly rounded float32 square root.  (__fsqrt_rn lowers to the native,
// approximate instruction in this toolchain; __builtin_sqrtf gets the correctly
// rounded expansion.)  Correct rounding makes it monotone, which the
// neighbour-list completeness test of the Boruvka shortcuts relies on, and
// makes every distance the same function of D2 in every kernel.
__device__ __forceinline__ float sqrt_rn(float x) { return __builtin_sqrtf(x); }

// one neighbour-list entry
struct __align__(8) Entry {
    float d2;
    int32_t idx;
};

// ---- kNN -----------------------------------------------------------------
enum KnnOut : int {
    kOutKnn = 1,     // final: out_idx / out_dist, first k entries
    kOutCore = 2,    // final: nbr lists (K = ms + 1) and core = sqrt(d2[ms-1]) (GEMM form; replaced by the
                     // direct-difference value of knn_core_kernel where the caller asks for core distances)
    kOutBound = 4,   // final: out_core[q] = D2 of entry k_out - 1 (the bound pass of the symmetric self-kNN)
};

struct KnnArgs {
    const float *Q;   // queries [d, *] (ld ldq); rows of the result
    int64_t ldq;
    int64_t q0;       // first query row of this chunk
    int64_t nq;       // rows in this chunk
    const float *nrm_q; // |q|^2, indexed by absolute row
    int64_t m;        // database points
    const float *nrm_b; // |b|^2 [m]
    int d;
    int self;         // Q == B: the pair (i, i) is forced to D2 = 0
    int64_t body_q;   // leading query tiles run whole (one workgroup, final lists)
    int splits;       // database splits of every later query tile
    int64_t tiles;    // ceil(m / TR)
    int out_mode;     // final form; split tiles write part[split][row - tail start][K]
    int k_out;        // entries written per row (k, or ms + 1 for core)
    int min_samples;  // core mode
    Entry *part;      // partial lists [splits][split-tile rows][K]
    int32_t *out_idx; // [n, k_out] absolute rows
    float *out_dist;  // [n, k_out] (kOutKnn) or d2 lists (kOutCore)
    float *out_core;  // [n]
    const float *Bt;  // database point-major [m, dp] (segment layout of tile_dim; the tiles and the direct differences read it)
    int dp;           // row stride of Bt: tile_dim(d)
    // query tiles to run (NULL: all): tile t = rows [t * gate_rows, (t + 1) * gate_rows) of the whole query set
    // runs when gate[t] != 0 (the merge kernel likewise skips the rows of the other tiles)
    const uint32_t *gate;
    int gate_rows;
    // symmetric self-kNN (knn_sym_kernel, sym_merge_kernel); Q and the database are the same n points
    const float *tau;     // per point: D2 of its k_out-th neighbour among a subset, a bound on the final one
    const float *theta;   // per point: tau widened for the column side's fast test
    Entry *colbuf;        // per point: colcap column-side candidates (D2, query index)
    uint32_t *colcnt;     // per point: candidates offered (may exceed colcap: then the list is recomputed)
    int colcap;
    uint32_t *gate_w;     // per query tile (gate_rows rows): set by sym_merge_kernel when a row's buffer overflowed
};

// Symmetric self-kNN (ekh_core_distances from kSymMinPoints points on): the
// bound pass runs the kNN against every kSymSubset-th point; the column
// buffers hold kSymColCap candidates per point.
constexpr int64_t kSymMinPoints = 16384;
constexpr int kSymSubset = 16;
constexpr int kSymColCap = 512;
// most database splits per query tile in the symmetric pass
constexpr int kSymMaxSplits = 16;

// host launchers (return hipError_t of the launch)
// Norms of X (into nx), of Y when ny is set, and Y's point-major copy when Bt is
// set, in one launch.
hipError_t launch_prep(const float *X, int64_t ldx, int64_t n, float *nx, const float *Y, int64_t ldy, int64_t m,
                       float *ny, float *Bt, int d, int dp, hipStream_t s);
hipError_t launch_knn_tile(int K, int QM, const KnnArgs &a, hipStream_t s);
hipError_t launch_knn_merge(int K, const KnnArgs &a, hipStream_t s);
hipError_t launch_knn_rescore(int K, const KnnArgs &a, hipStream_t s);
hipError_t launch_knn_core(int K, const KnnArgs &a, hipStream_t s);
// symmetric pass: grid = query tiles x a.splits, query tile t over database
// tiles [t * QT / TR, a.tiles) in a.splits pieces
hipError_t launch_knn_sym(int K, int QM, const KnnArgs &a, hipStream_t s);
hipError_t launch_sym_merge(int K, const KnnArgs &a, hipStream_t s);
// rows 0, step, 2 step, ... of the point-major copy bt [n, dp] and their norms into bs, ns
hipError_t launch_subset_gather(const float *bt, const float *nx, int64_t n, int dp, int step, float *bs, float *ns,
                                hipStream_t s);
// theta = tau widened for the column side's fast test (from tau and the norms); zeroes colcnt [n] and gate [ntiles]
hipError_t launch_sym_setup(const float *tau, const float *nx, int64_t n, float *theta, uint32_t *colcnt,
                            uint32_t *gate, int64_t ntiles, hipStream_t s);

// ---- Boruvka ---------------------------------------------------------------
constexpr uint64_t kNoEdge = ~0ull;
constexpr uint32_t kInfBits = 0x7f800000u;

struct BvCounters {
    uint32_t n_active;
    uint32_t n_resolved;
    uint32_t n_skipped;
    uint32_t n_edges;
    uint32_t n_roots;
    uint32_t n_missing;
    uint32_t n_active_g; // active points of the largest component, listed apart
    uint32_t n_comp_g;   // points outside it, gathered for their scan
    uint64_t giant;      // size << 32 | label of the largest component
};

struct ScanArgs {
    // query side (the active points index these)
    const float *X;
    int64_t ldx;
    int64_t n;
    const float *nrm;     // |x|^2 [n]
    const float *core;    // [n]
    const int32_t *comp;  // component label of every point
    // database side, point-major rows [nb, dp] (segment layout of tile_dim):
    // all points, or a gathered subset whose row j is point orig[j]
    const float *Xb;
    int dp;
    int64_t nb;
    const float *nrm_b;
    const float *core_b;
    const int32_t *comp_b;
    const int32_t *orig;  // NULL: row j is point j
    const uint32_t *compW; // bound W bits per component (kInfBits = none)
    const int32_t *act;   // active points
    const uint32_t *nact; // their number, read on the device (set by the activity pass)
    uint64_t *best;       // per-point best key (W bits << 32 | partner), atomicMin
    int d;
    int64_t tiles;        // database tiles
};
// Database tiles per split of the scan, at least (the split count is chosen on
// the device, where the number of active points is known).
constexpr int64_t kScanMinTilesPerSplit = 4;

// grid: workgroups launched (normally one round of resident ones); they walk
// the (query tile, database split) items the device-side count implies
hipError_t launch_scan_tile(int QM, const ScanArgs &a, int64_t grid, hipStream_t s);

struct BvState {
    int64_t n;
    int K;           // list length (min_samples + 1)
    const int32_t *nbr_idx;
    const float *nbr_d2;
    const float *core;
    int32_t *comp;
    uint64_t *cc;      // per point (comp << 32 | core bits): one gather per list entry
    int32_t *parent;
    int32_t *act;
    uint8_t *resolved;
    float *lbound;     // per point: no edge of it is lighter (from its core and list)
    uint64_t *best;
    uint64_t *cmin1;   // per component (W bits << 32 | lo)
    uint32_t *cmin2;   // per component hi
    uint32_t *compW;   // per component bound W bits
    uint32_t *csize;   // per component size (zero between rounds)
    int32_t *act_g;    // active points of the largest component
    int32_t *e_lo;
    int32_t *e_hi;
    float *e_w;
    BvCounters *ctr;
};

hipError_t bv_init(const BvState &st, hipStream_t s);
hipError_t bv_reset_counters(const BvState &st, hipStream_t s);
hipError_t bv_candidates(const BvState &st, int use_neighbour_edges, int use_bound, hipStream_t s);
hipError_t bv_select_active(const BvState &st, int use_bound, int split_giant, hipStream_t s);
hipError_t bv_giant(const BvState &st, hipStream_t s);
hipError_t bv_complement(const BvState &st, int32_t giant, int32_t *orig, hipStream_t s);
// rows orig[0 .. ns) of the point-major copy P [n, dp] into xs [ns, dp], with their norms, core distances and labels
hipError_t bv_gather_points(const float *P, int dp, const int32_t *orig, int64_t ns, const float *nrm,
                            const float *core, const int32_t *comp, float *xs, float *nrm_s, float *core_s,
                            int32_t *comp_s, const uint32_t *count, const uint32_t *gate, hipStream_t s);
hipError_t bv_component_min(const BvState &st, hipStream_t s);
hipError_t bv_select_edges(const BvState &st, hipStream_t s);
hipError_t bv_jump(const BvState &st, hipStream_t s);
hipError_t bv_relabel(const BvState &st, hipStream_t s);

// reported edge weights by direct differences (P: point-major copy [n, dp])
hipError_t bv_edge_weights(const float *P, int dp, const float *core, const int32_t *lo, const int32_t *hi, int64_t ne,
                           int64_t n, float *w, hipStream_t s);

// final edge order (W, lo, hi)
size_t edge_sort_temp_bytes(int64_t ne);
hipError_t edge_sort(const int32_t *lo, const int32_t *hi, const float *w, int64_t ne, void *tmp, size_t tmp_bytes,
                     uint32_t *u32a, uint32_t *u32b, uint32_t *u32c, uint32_t *u32d, uint64_t *u64a, uint64_t *u64b,
                     int32_t *out_lo, int32_t *out_hi, float *out_w, hipStream_t s);

} // namespace ekh
