// Dense tile kernels of libekh on gfx950, part 2: norms, the kNN dispatch over
// list lengths, and the Boruvka cheapest-edge scan.  The shared tile loop and
// the kNN kernels are in tile_common.h / knn_inst.hip.
#include "tile_common.h"

namespace ekh {

// ---------------------------------------------------------------- norms
// |x_i|^2 as the diagonal of a 16 x 16 Gram block computed by the same MFMA
// chain as the tile kernels (same feature order, same k-step sequence, starting
// from 0).  So the norm of x equals, bit for bit, the dot product the tile
// kernels compute for x against any bitwise-identical point, and identical
// points get D2 = fma(-2, n, 2n) = 0 exactly.  64 points per workgroup (16 per
// wave); qs = the k-step count QM of the tile kernels for this d.
__device__ __forceinline__ void norms_block(const float *__restrict__ X, int64_t ldx, int64_t n, int d, int qs,
                                            float *__restrict__ out, int64_t block) {
    const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
    const int64_t p = (block * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 16 + li;
    const bool valid = p < n;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < qs; ++s) {
        const int f = g * qs + s;
        const float v = (valid && f < d) ? X[(int64_t)f * ldx + p] : 0.f;
        acc = mfma16(v, v, acc);
    }
    // lane (g, i) holds rows 4g..4g+3 of column i: the diagonal entry (i, i)
    // sits in the lane with g = i / 4, element i % 4
    if (valid && (li >> 2) == g) out[p] = acc[li & 3];
}

// Point-major copy of a feature-major point set, for tiles and gathers of
// whole points: Bt[j * dp + p] = B[f * ldb + j] for the feature f at position p
// (pm_feature), 0 at the positions that hold none.  One 32-position x
// 32-point tile per workgroup, through LDS (one padding column), coalesced on
// both sides.
__device__ __forceinline__ void point_major_block(const float *__restrict__ B, int64_t ldb, int64_t m, int d, int qm,
                                                  int dp, float *__restrict__ Bt, int64_t bx, int by) {
    __shared__ float t[32][33];
    const int64_t j0 = bx * 32;
    const int p0 = by * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int r = ty; r < 32; r += 8) {
        const int f = pm_feature(p0 + r, qm, d);
        const int64_t j = j0 + tx;
        t[r][tx] = (f >= 0 && j < m) ? B[(int64_t)f * ldb + j] : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
        const int64_t j = j0 + r;
        const int p = p0 + tx;
        if (j < m && p < dp) Bt[j * dp + p] = t[tx][r];
    }
}

namespace {
constexpr int kNormPoints = 64; // points per norms workgroup
int64_t norm_blocks(int64_t n) { return (n + kNormPoints - 1) / kNormPoints; }

// The preparation of one kNN call in a single launch: norms of the queries,
// norms of the database (unless it is the query set), and the database's
// point-major copy (when Bt is set).  The workgroup index picks the part.
struct PrepArgs {
    const float *X, *Y;
    int64_t ldx, n, ldy, m;
    float *nx, *ny, *Bt;
    int d, dp, qm;
    int64_t bx, by, tiles_x; // workgroups of the X norms, of the Y norms; point-major tiles per feature block
};

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    const int64_t b = blockIdx.x;
    if (b < a.bx) {
        norms_block(a.X, a.ldx, a.n, a.d, a.qm, a.nx, b);
    } else if (b < a.bx + a.by) {
        norms_block(a.Y, a.ldy, a.m, a.d, a.qm, a.ny, b - a.bx);
    } else {
        const int64_t t = b - a.bx - a.by;
        point_major_block(a.Y, a.ldy, a.m, a.d, a.qm, a.dp, a.Bt, t % a.tiles_x, (int)(t / a.tiles_x));
    }
}
} // namespace

hipError_t launch_prep(const float *X, int64_t ldx, int64_t n, float *nx, const float *Y, int64_t ldy, int64_t m,
                       float *ny, float *Bt, int d, int dp, hipStream_t s) {
    PrepArgs a{};
    a.X = X;
    a.Y = Y;
    a.ldx = ldx;
    a.n = n;
    a.ldy = ldy;
    a.m = m;
    a.nx = nx;
    a.ny = ny;
    a.Bt = Bt;
    a.d = d;
    a.dp = dp;
    a.qm = pick_qm(d);
    if (dp != tile_dim(d)) return hipErrorInvalidValue;
    a.bx = nx ? norm_blocks(n) : 0;
    a.by = ny ? norm_blocks(m) : 0;
    a.tiles_x = (m + 31) / 32;
    const int64_t pm = Bt ? a.tiles_x * ((dp + 31) / 32) : 0;
    const int64_t blocks = a.bx + a.by + pm;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}


// ---------------------------------------------------------------- kNN dispatch
hipError_t launch_knn_tile(int K, int QM, const KnnArgs &a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    switch (K) {
    case 2: return launch_knn_tile_k<2>(QM, a, s);
    case 4: return launch_knn_tile_k<4>(QM, a, s);
    case 8: return launch_knn_tile_k<8>(QM, a, s);
    case 10: return launch_knn_tile_k<10>(QM, a, s);
    case 11: return launch_knn_tile_k<11>(QM, a, s);
    case 16: return launch_knn_tile_k<16>(QM, a, s);
    case 32: return launch_knn_tile_k<32>(QM, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_knn_sym(int K, int QM, const KnnArgs &a, hipStream_t s) {
    switch (K) {
    case 2: return launch_knn_sym_k<2>(QM, a, s);
    case 4: return launch_knn_sym_k<4>(QM, a, s);
    case 8: return launch_knn_sym_k<8>(QM, a, s);
    case 10: return launch_knn_sym_k<10>(QM, a, s);
    case 11: return launch_knn_sym_k<11>(QM, a, s);
    case 16: return launch_knn_sym_k<16>(QM, a, s);
    case 32: return launch_knn_sym_k<32>(QM, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sym_merge(int K, const KnnArgs &a, hipStream_t s) {
    switch (K) {
    case 2: return launch_sym_merge_k<2>(a, s);
    case 4: return launch_sym_merge_k<4>(a, s);
    case 8: return launch_sym_merge_k<8>(a, s);
    case 10: return launch_sym_merge_k<10>(a, s);
    case 11: return launch_sym_merge_k<11>(a, s);
    case 16: return launch_sym_merge_k<16>(a, s);
    case 32: return launch_sym_merge_k<32>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// One thread per 16-byte piece of a gathered row.
__global__ __launch_bounds__(256) void subset_gather_kernel(const float *__restrict__ bt, const float *__restrict__ nx,
                                                            int64_t ns, int dp, int step, float *__restrict__ bs,
                                                            float *__restrict__ nrm_s) {
    const int pieces = dp / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= ns * pieces) return;
    const int64_t r = gid / pieces;
    const int c = (int)(gid % pieces);
    const int64_t src = r * step;
    reinterpret_cast<f4 *>(bs + r * dp)[c] = reinterpret_cast<const f4 *>(bt + src * dp)[c];
    if (c == 0) nrm_s[r] = nx[src];
}

hipError_t launch_subset_gather(const float *bt, const float *nx, int64_t n, int dp, int step, float *bs, float *ns,
                                hipStream_t s) {
    if (step < 1 || dp % 4) return hipErrorInvalidValue;
    const int64_t rows = (n + step - 1) / step;
    const int64_t threads = rows * (dp / 4);
    if ((threads + 255) / 256 > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(subset_gather_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, bt, nx, rows,
                       dp, step, bs, ns);
    return hipGetLastError();
}

// theta = tau + 2^-19 (n + tau) (see the symmetric pass's column side), and
// the zeroed counters of one call
__global__ __launch_bounds__(256) void sym_setup_kernel(const float *__restrict__ tau, const float *__restrict__ nx,
                                                        int64_t n, float *__restrict__ theta,
                                                        uint32_t *__restrict__ colcnt, uint32_t *__restrict__ gate,
                                                        int64_t ntiles) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const float t = tau[i];
        theta[i] = fmaf(nx[i] + t, 1.0f / 524288.0f, t);
        colcnt[i] = 0u;
    }
    if (i < ntiles) gate[i] = 0u;
}

hipError_t launch_sym_setup(const float *tau, const float *nx, int64_t n, float *theta, uint32_t *colcnt,
                            uint32_t *gate, int64_t ntiles, hipStream_t s) {
    const int64_t m = n > ntiles ? n : ntiles;
    hipLaunchKernelGGL(sym_setup_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, tau, nx, n, theta, colcnt,
                       gate, ntiles);
    return hipGetLastError();
}

hipError_t launch_knn_rescore(int K, const KnnArgs &a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    switch (K) {
    case 2: return launch_knn_rescore_k<2>(a, s);
    case 4: return launch_knn_rescore_k<4>(a, s);
    case 8: return launch_knn_rescore_k<8>(a, s);
    case 10: return launch_knn_rescore_k<10>(a, s);
    case 11: return launch_knn_rescore_k<11>(a, s);
    case 16: return launch_knn_rescore_k<16>(a, s);
    case 32: return launch_knn_rescore_k<32>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_knn_core(int K, const KnnArgs &a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    switch (K) {
    case 2: return launch_knn_core_k<2>(a, s);
    case 4: return launch_knn_core_k<4>(a, s);
    case 8: return launch_knn_core_k<8>(a, s);
    case 10: return launch_knn_core_k<10>(a, s);
    case 11: return launch_knn_core_k<11>(a, s);
    case 16: return launch_knn_core_k<16>(a, s);
    case 32: return launch_knn_core_k<32>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_knn_merge(int K, const KnnArgs &a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    switch (K) {
    case 2: return launch_knn_merge_k<2>(a, s);
    case 4: return launch_knn_merge_k<4>(a, s);
    case 8: return launch_knn_merge_k<8>(a, s);
    case 10: return launch_knn_merge_k<10>(a, s);
    case 11: return launch_knn_merge_k<11>(a, s);
    case 16: return launch_knn_merge_k<16>(a, s);
    case 32: return launch_knn_merge_k<32>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- Boruvka scan
// Cheapest edge from each active point a to another component, over all n
// points ("HDBSCAN" page, "Exact shortcuts": the points the shortcuts did not
// settle are the only ones compared with every other point).  Key of an edge seen from a: (W bits << 32 | b);
// for a fixed a this order equals the edge order (W, lower, higher index).

// A squared-distance threshold that no improving candidate can exceed: an
// improving b has sqrt_rn(D2) <= W <= W*, hence D2 <= W*^2 (1 + 2^-23 + ...),
// below W*^2 (1 + 2^-20) even after the two roundings of this product.
__device__ __forceinline__ float scan_threshold(float w) {
    if (w < 1e-18f) return 1e-36f;
    const float t = w * w * 1.00000095367431640625f;
    return t < FLT_MAX ? t : FLT_MAX;
}

// Fast test per element, as in the kNN epilogue: t = fma(-2, s, nb) against
// thq = thr - na, widened by 2^-20 (thr + na).  Every element whose D2 =
// fma(-2, s, na + nb) is <= thr has t <= thq (the rounding errors between D2
// and t + na are a few units of 2^-24 (na + nb + thr), and nb <= 2 na + 2 thr
// for such an element), so the test never skips a candidate; the exact D2
// decides in candidate().
template <int CB, int RB> struct EpiScan {
    uint64_t best[CB];
    uint64_t init[CB];
    float thr[CB];
    float thq[CB];
    float na[CB];
    float corea[CB];
    int32_t ca[CB];
    int g;
    const int32_t *orig; // database row -> point (NULL: the same)

    __device__ __forceinline__ void candidate(int cb, float d2, int32_t j, int32_t cj, float corej) {
        // same component, or a padding row past the database (label -1)
        if (cj == ca[cb] || cj < 0) return;
        const float D = sqrt_rn(d2 > 0.f ? d2 : 0.f);
        const float W = fmaxf(fmaxf(corea[cb], corej), D);
        const uint32_t b = orig ? (uint32_t)orig[j] : (uint32_t)j;
        const uint64_t key = ((uint64_t)__float_as_uint(W) << 32) | b;
        if (key < best[cb]) {
            best[cb] = key;
            set_threshold(cb, scan_threshold(W));
        }
    }
    __device__ __forceinline__ void set_threshold(int cb, float t) {
        constexpr float kWiden = 1.0f / 1048576.0f;
        thr[cb] = t;
        thq[cb] = fmaf(t, 1.0f + kWiden, -na[cb] * (1.0f - kWiden));
    }
    __device__ __forceinline__ void tile(const f4 (&acc)[RB][CB], const float *nrm, const int32_t *comp,
                                         const float *core, int64_t j0) {
        f4 nb4[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) nb4[rb] = *reinterpret_cast<const f4 *>(nrm + rb * 16 + 4 * g);
        bool hit = false;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            float mn = INFINITY;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mn = fminf(mn, fmaf(-2.f, acc[rb][cb][r], nb4[rb][r]));
            hit |= mn <= thq[cb];
        }
        if (!hit) return;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rb * 16 + 4 * g + r;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const float d2 = fmaf(-2.f, acc[rb][cb][r], na[cb] + nb4[rb][r]);
                    if (d2 <= thr[cb]) candidate(cb, d2, (int32_t)(j0 + row), comp[row], core[row]);
                }
            }
    }
};

template <int QM>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(scan_waves_per_simd(QM), scan_waves_per_simd(QM))))
void scan_tile_kernel(ScanArgs a) {
    constexpr int CB = scan_col_blocks(QM);
    using T = Tile<QM>;
    constexpr int QT = kWaves * 16 * CB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
    // The number of active points is known only here (the host does not wait
    // for it): q query tiles, each in sp database splits, as many as fill the
    // launched workgroups once (the scan has no list warm-up), at least
    // kScanMinTilesPerSplit tiles each.  Workgroup w takes items w, w + grid,
    // ... (item = split * q + query tile), a loop every workgroup leaves after
    // at most ceil(items / grid) trips.
    const int64_t nact = (int64_t)__hip_atomic_load(a.nact, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t q = (nact + QT - 1) / QT;
    if (q == 0) return;
    const int64_t G = gridDim.x;
    int64_t sp = q < G ? G / q : 1;
    const int64_t smax = a.tiles / kScanMinTilesPerSplit;
    sp = sp < smax ? sp : (smax > 1 ? smax : 1);
    const int64_t items = q * sp;
    for (int64_t it = blockIdx.x; it < items; it += G) {
        const int64_t qt = it % q;
        const int64_t split = it / q;
        const int64_t cbase = qt * QT;

        EpiScan<CB, T::RB> epi;
        epi.g = g;
        epi.orig = a.orig;
        float bq[CB][QM];
        int32_t pt[CB];
        bool valid[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int64_t c = cbase + wave * 16 * CB + cb * 16 + li;
            valid[cb] = c < nact;
            const int32_t p = valid[cb] ? a.act[c] : 0;
            pt[cb] = p;
            load_query<QM>(a.X, a.ldx, p, valid[cb], a.d, g, bq[cb]);
            epi.na[cb] = a.nrm[p];
            epi.corea[cb] = a.core[p];
            epi.ca[cb] = a.comp[p];
            // start from the best edge already known for this point's component
            float w0 = __uint_as_float(a.compW[epi.ca[cb]]);
            const uint64_t own = a.best[p];
            if (own != kNoEdge) w0 = fminf(w0, __uint_as_float((uint32_t)(own >> 32)));
            epi.init[cb] = ((uint64_t)__float_as_uint(w0) << 32) | 0xffffffffull;
            epi.best[cb] = epi.init[cb];
            epi.set_threshold(cb, (!valid[cb] || epi.corea[cb] > w0) ? -INFINITY : scan_threshold(w0));
        }
        const int64_t tb = a.tiles * split / sp, te = a.tiles * (split + 1) / sp;
        run_tiles<QM, CB, true, 1>(a.Xb, (int32_t)a.nb, a.nrm_b, a.comp_b, a.core_b, (int32_t)tb, (int32_t)te, bq, epi);

#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            uint64_t b = epi.best[cb];
#pragma unroll
            for (int mask = 16; mask <= 32; mask <<= 1) {
                const uint32_t lo = __shfl_xor((uint32_t)b, mask), hi = __shfl_xor((uint32_t)(b >> 32), mask);
                const uint64_t o = ((uint64_t)hi << 32) | lo;
                b = o < b ? o : b;
            }
            if (g == 0 && valid[cb] && b < epi.init[cb])
                atomicMin((unsigned long long *)&a.best[pt[cb]], (unsigned long long)b);
        }
    }
}

template <int QM> static hipError_t scan_launch(const ScanArgs &a, int64_t grid, hipStream_t s) {
    if (a.dp != tile_dim(a.d) || pick_qm(a.d) != QM) return hipErrorInvalidValue;
    hipLaunchKernelGGL((scan_tile_kernel<QM>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_scan_tile(int QM, const ScanArgs &a, int64_t grid, hipStream_t s) {
    if (grid <= 0 || grid > 0x7fffffff || a.tiles <= 0) return hipErrorInvalidValue;
    switch (QM) {
#define EKH_SCAN_CASE(q)                                                                                               \
    case q: return scan_launch<q>(a, grid, s);
        EKH_FOR_EACH_QM(EKH_SCAN_CASE)
#undef EKH_SCAN_CASE
    default: return hipErrorInvalidValue;
    }
}

} // namespace ekh
