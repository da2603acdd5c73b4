// Dense tile kernels of libekh on gfx950: kNN tile (MFMA distances + register
// top-K) and the Boruvka cheapest-edge scan tile.
//
// Distances follow the clustering page, "k-nearest neighbours are a matrix
// product": D2 = (|q|^2 + |b|^2) - 2 q.b, the q.b contraction being one dense
// product that is never materialised: each 16 x 16 block of it lives in the
// accumulator registers of v_mfma_f32_16x16x4_f32 and is consumed there.
//
// MFMA 16x16x4 f32 lane layout (lane = 16 * g + i, g = 0..3, i = 0..15):
//   A operand: lane holds A[i][g]    (database row i, feature 4s + g of k-step s)
//   B operand: lane holds B[g][i]    (feature 4s + g of query column i)
//   result   : lane holds C[4g + r][i], r = 0..3
// so a lane owns one query column and sees database rows 4g..4g+3 of every
// 16-row block, in ascending order; four lanes (g = 0..3) share a column.
#include "ekh_internal.h"

#include <float.h>
#include <math.h>

namespace ekh {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma16(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- norms
// |x_i|^2 accumulated feature by feature with fmaf, in one fixed order; every
// entry point uses this kernel so D2 is the same function everywhere.
__global__ void norms_kernel(const float *__restrict__ X, int64_t ldx, int64_t n, int d, float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int f = 0; f < d; ++f) {
        const float v = X[(int64_t)f * ldx + i];
        s = fmaf(v, v, s);
    }
    out[i] = s;
}

hipError_t launch_norms(const float *X, int64_t ldx, int64_t n, int d, float *out, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int bs = 256;
    hipLaunchKernelGGL(norms_kernel, dim3((unsigned)((n + bs - 1) / bs)), dim3(bs), 0, s, X, ldx, n, d, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------- tile loop
template <int QM, int CB> struct Tile {
    static constexpr int TR = TileGeo<QM>::TR; // database rows per tile
    static constexpr int RB = TR / 16;         // 16-row blocks per tile
    static constexpr int TRS = TR + 16;        // LDS row stride: lane groups g land on distinct banks
    static constexpr int FD = QM * 4;          // features held (d <= FD)
    static constexpr int FSTEP = kThreads / TR; // feature rows per load pass
    static constexpr int PF = FD / FSTEP;      // prefetch registers per thread
    static_assert(FD % FSTEP == 0, "tile shape");
};

// Streams database tiles [t_begin, t_end) through a double-buffered LDS tile
// and hands each 16 x 16 result block set to epi.tile().  PAYLOAD also stages
// the per-row component label and core distance for the scan epilogue.
template <int QM, int CB, bool PAYLOAD, class Epi>
__device__ __forceinline__ void run_tiles(const float *__restrict__ B, int64_t ldb, int64_t m,
                                          const float *__restrict__ nrm_b, const int32_t *__restrict__ comp_b,
                                          const float *__restrict__ core_b, int d, int chunks, int64_t t_begin,
                                          int64_t t_end, const float (&bq)[CB][QM], Epi &epi) {
    using T = Tile<QM, CB>;
    __shared__ float sm_tile[2][T::FD * T::TRS];
    __shared__ __align__(16) float sm_nrm[2][T::TR];
    __shared__ int32_t sm_comp[2][PAYLOAD ? T::TR : 1];
    __shared__ float sm_core[2][PAYLOAD ? T::TR : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int lrow = tid % T::TR, lf0 = tid / T::TR;
    const int fused = chunks * 16;

    float pf[T::PF];
    float pn = 0.f, pcore = 0.f;
    int32_t pcomp = -1;

    auto load = [&](int64_t t) {
        const int64_t j = t * T::TR + lrow;
        const bool jv = j < m;
#pragma unroll
        for (int p = 0; p < T::PF; ++p) {
            const int f = lf0 + p * T::FSTEP;
            pf[p] = (jv && f < d) ? B[(int64_t)f * ldb + j] : 0.f;
        }
        if (tid < T::TR) {
            const int64_t jj = t * T::TR + tid;
            const bool v = jj < m;
            pn = v ? nrm_b[jj] : INFINITY; // padding rows never qualify
            if (PAYLOAD) {
                pcomp = v ? comp_b[jj] : -1;
                pcore = v ? core_b[jj] : INFINITY;
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int p = 0; p < T::PF; ++p) {
            const int f = lf0 + p * T::FSTEP;
            if (f < fused) sm_tile[buf][f * T::TRS + lrow] = pf[p];
        }
        if (tid < T::TR) {
            sm_nrm[buf][tid] = pn;
            if (PAYLOAD) {
                sm_comp[buf][tid] = pcomp;
                sm_core[buf][tid] = pcore;
            }
        }
    };

    if (t_begin < t_end) {
        load(t_begin);
        store(0);
    }
    __syncthreads();
    int buf = 0;
    for (int64_t t = t_begin; t < t_end; ++t) {
        const bool more = t + 1 < t_end;
        if (more) load(t + 1);
        f4 acc[T::RB][CB];
#pragma unroll
        for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f4{0.f, 0.f, 0.f, 0.f};
        const float *tl = sm_tile[buf];
#pragma unroll
        for (int c = 0; c < QM / 4; ++c) {
            if (c < chunks) {
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int s = c * 4 + s4;
                    float a[T::RB];
#pragma unroll
                    for (int rb = 0; rb < T::RB; ++rb) a[rb] = tl[(4 * s + g) * T::TRS + rb * 16 + li];
#pragma unroll
                    for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mfma16(a[rb], bq[cb][s], acc[rb][cb]);
                }
            }
        }
        if (PAYLOAD)
            epi.tile(acc, sm_nrm[buf], sm_comp[buf], sm_core[buf], t * T::TR);
        else
            epi.tile(acc, sm_nrm[buf], nullptr, nullptr, t * T::TR);
        if (more) store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
}

// Loads the register-resident query operand: lane (g, i) holds feature 4s + g
// of its query column for every k-step s.
template <int QM>
__device__ __forceinline__ void load_query(const float *__restrict__ Q, int64_t ldq, int64_t col, bool valid, int d,
                                           int g, float (&bq)[QM]) {
#pragma unroll
    for (int s = 0; s < QM; ++s) {
        const int f = 4 * s + g;
        bq[s] = (valid && f < d) ? Q[(int64_t)f * ldq + col] : 0.f;
    }
}

// ---------------------------------------------------------------- top-K list
// Sorted ascending list of K (d2, idx) entries in registers.  Insertion is the
// fixed, compile-time-unrolled compare-and-swap sequence of the HDBSCAN page
// ("The hang"): the candidate replaces the last entry and moves towards the
// front through K - 1 conditional swaps, with no data-dependent loop.
template <int K> struct TopK {
    float d[K];
    int32_t i[K];

    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int t = 0; t < K; ++t) {
            d[t] = INFINITY;
            i[t] = 0x7fffffff;
        }
    }
    // Candidate from a stream whose indices ascend: it is larger than every
    // entry in index, so a strict '<' on d2 keeps equal distances in index order.
    __device__ __forceinline__ void push_ascending(float v, int32_t j) {
        d[K - 1] = v;
        i[K - 1] = j;
#pragma unroll
        for (int t = K - 1; t > 0; --t) {
            const bool sw = d[t] < d[t - 1];
            const float a = sw ? d[t] : d[t - 1], b = sw ? d[t - 1] : d[t];
            const int32_t ia = sw ? i[t] : i[t - 1], ib = sw ? i[t - 1] : i[t];
            d[t - 1] = a;
            d[t] = b;
            i[t - 1] = ia;
            i[t] = ib;
        }
    }
    __device__ __forceinline__ static bool less(float a, int32_t ia, float b, int32_t ib) {
        return a < b || (a == b && ia < ib);
    }
    // Candidate in any order: full (d2, idx) comparison.
    __device__ __forceinline__ void push_any(float v, int32_t j) {
        if (!less(v, j, d[K - 1], i[K - 1])) return;
        d[K - 1] = v;
        i[K - 1] = j;
#pragma unroll
        for (int t = K - 1; t > 0; --t) {
            const bool sw = less(d[t], i[t], d[t - 1], i[t - 1]);
            const float a = sw ? d[t] : d[t - 1], b = sw ? d[t - 1] : d[t];
            const int32_t ia = sw ? i[t] : i[t - 1], ib = sw ? i[t - 1] : i[t];
            d[t - 1] = a;
            d[t] = b;
            i[t - 1] = ia;
            i[t] = ib;
        }
    }
    // Merge with the list held by lane (lane ^ mask); both lanes end equal.
    __device__ __forceinline__ void merge_xor(int mask) {
        float od[K];
        int32_t oi[K];
#pragma unroll
        for (int t = 0; t < K; ++t) {
            od[t] = __shfl_xor(d[t], mask);
            oi[t] = __shfl_xor(i[t], mask);
        }
#pragma unroll
        for (int t = 0; t < K; ++t) push_any(od[t], oi[t]);
    }
};

// ---------------------------------------------------------------- kNN epilogue
template <int K, int CB, int RB> struct EpiKnn {
    TopK<K> L[CB];
    float nq[CB];
    int32_t qrow[CB];
    int64_t qlo, qhi; // absolute query rows of this workgroup, for the self diagonal
    int self;
    int g;

    __device__ __forceinline__ void tile(const f4 (&acc)[RB][CB], const float *nrm, const int32_t *, const float *,
                                         int64_t j0) {
        const bool diag = self && (j0 < qhi) && (j0 + RB * 16 > qlo);
        if (diag) {
            tile_impl<true>(acc, nrm, j0);
        } else {
            tile_impl<false>(acc, nrm, j0);
        }
    }
    template <bool DIAG>
    __device__ __forceinline__ void tile_impl(const f4 (&acc)[RB][CB], const float *nrm, int64_t j0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const f4 nb4 = *reinterpret_cast<const f4 *>(nrm + rb * 16 + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int32_t j = (int32_t)(j0 + rb * 16 + 4 * g + r);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    float d2 = fmaf(-2.f, acc[rb][cb][r], nq[cb] + nb4[r]);
                    if (DIAG && j == qrow[cb]) d2 = 0.f;
                    if (d2 < L[cb].d[K - 1]) L[cb].push_ascending(d2 > 0.f ? d2 : 0.f, j);
                }
            }
        }
    }
};

// Writes a finished list for absolute row q.
template <int K>
__device__ __forceinline__ void write_list(const KnnArgs &a, const TopK<K> &L, int64_t q, int split) {
    if (a.out_mode == kOutPartial) {
        Entry *dst = a.part + ((int64_t)split * a.nq + (q - a.q0)) * K;
#pragma unroll
        for (int t = 0; t < K; ++t) dst[t] = Entry{L.d[t], L.i[t]};
    } else if (a.out_mode == kOutKnn) {
#pragma unroll
        for (int t = 0; t < K; ++t) {
            if (t < a.k_out) {
                if (a.out_idx) a.out_idx[q * a.k_out + t] = L.i[t];
                if (a.out_dist) a.out_dist[q * a.k_out + t] = sqrt_rn(L.d[t]);
            }
        }
    } else {
        float c = 0.f;
#pragma unroll
        for (int t = 0; t < K; ++t) {
            if (t == a.min_samples - 1) c = L.d[t];
            if (t < a.k_out) {
                if (a.out_idx) a.out_idx[q * a.k_out + t] = L.i[t];
                if (a.out_dist) a.out_dist[q * a.k_out + t] = L.d[t];
            }
        }
        a.out_core[q] = sqrt_rn(c);
    }
}

template <int K, int QM>
__global__ __launch_bounds__(kThreads) void knn_tile_kernel(KnnArgs a) {
    constexpr int CB = knn_col_blocks(K, QM);
    using T = Tile<QM, CB>;
    constexpr int QT = kWaves * 16 * CB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
    const int split = blockIdx.y;
    const int64_t qbase = (int64_t)blockIdx.x * QT; // local row of the workgroup's first query

    EpiKnn<K, CB, T::RB> epi;
    float bq[CB][QM];
    bool qv[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t ql = qbase + wave * 16 * CB + cb * 16 + li;
        qv[cb] = ql < a.nq;
        const int64_t q = a.q0 + (qv[cb] ? ql : 0);
        load_query<QM>(a.Q, a.ldq, q, qv[cb], a.d, g, bq[cb]);
        epi.nq[cb] = qv[cb] ? a.nrm_q[q] : 0.f;
        epi.qrow[cb] = (int32_t)(a.q0 + ql);
        epi.L[cb].clear();
    }
    epi.qlo = a.q0 + qbase;
    epi.qhi = a.q0 + (qbase + QT < a.nq ? qbase + QT : a.nq);
    epi.self = a.self;
    epi.g = g;

    const int64_t tb = a.tiles * split / a.splits, te = a.tiles * (split + 1) / a.splits;
    run_tiles<QM, CB, false>(a.B, a.ldb, a.m, a.nrm_b, nullptr, nullptr, a.d, a.chunks, tb, te, bq, epi);

    // merge the four lane groups that share each query column
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        epi.L[cb].merge_xor(16);
        epi.L[cb].merge_xor(32);
    }
    if (g == 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            if (qv[cb]) write_list<K>(a, epi.L[cb], epi.qrow[cb], split);
    }
}

// One thread per row: merges the split lists in split order.
template <int K> __global__ void knn_merge_kernel(KnnArgs a) {
    const int64_t ql = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (ql >= a.nq) return;
    TopK<K> L;
    L.clear();
    for (int s = 0; s < a.splits; ++s) {
        const Entry *src = a.part + ((int64_t)s * a.nq + ql) * K;
#pragma unroll
        for (int t = 0; t < K; ++t) {
            const Entry e = src[t];
            L.push_any(e.d2, e.idx);
        }
    }
    write_list<K>(a, L, a.q0 + ql, 0); // a.out_mode is the final mode here
}

template <int K, int QM> static hipError_t knn_tile_launch(const KnnArgs &a, hipStream_t s) {
    constexpr int CB = knn_col_blocks(K, QM);
    constexpr int QT = kWaves * 16 * CB;
    const dim3 grid((unsigned)((a.nq + QT - 1) / QT), (unsigned)a.splits);
    hipLaunchKernelGGL((knn_tile_kernel<K, QM>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int K> static hipError_t knn_tile_qm(int QM, const KnnArgs &a, hipStream_t s) {
    switch (QM) {
    case 16: return knn_tile_launch<K, 16>(a, s);
    case 32: return knn_tile_launch<K, 32>(a, s);
    case 64: return knn_tile_launch<K, 64>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_knn_tile(int K, int QM, const KnnArgs &a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    switch (K) {
    case 2: return knn_tile_qm<2>(QM, a, s);
    case 4: return knn_tile_qm<4>(QM, a, s);
    case 8: return knn_tile_qm<8>(QM, a, s);
    case 11: return knn_tile_qm<11>(QM, a, s);
    case 16: return knn_tile_qm<16>(QM, a, s);
    case 32: return knn_tile_qm<32>(QM, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_knn_merge(int K, const KnnArgs &a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    const int bs = 256;
    const dim3 grid((unsigned)((a.nq + bs - 1) / bs));
    switch (K) {
    case 2: hipLaunchKernelGGL(knn_merge_kernel<2>, grid, dim3(bs), 0, s, a); break;
    case 4: hipLaunchKernelGGL(knn_merge_kernel<4>, grid, dim3(bs), 0, s, a); break;
    case 8: hipLaunchKernelGGL(knn_merge_kernel<8>, grid, dim3(bs), 0, s, a); break;
    case 11: hipLaunchKernelGGL(knn_merge_kernel<11>, grid, dim3(bs), 0, s, a); break;
    case 16: hipLaunchKernelGGL(knn_merge_kernel<16>, grid, dim3(bs), 0, s, a); break;
    case 32: hipLaunchKernelGGL(knn_merge_kernel<32>, grid, dim3(bs), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- Boruvka scan
// Cheapest edge from each active point a to another component, over all n
// points ("HDBSCAN" page, "Exact shortcuts": only the remaining clips are
// scanned against all others).  Key of an edge seen from a: (W bits << 32 | b);
// for a fixed a this order equals the edge order (W, lower, higher index).

// A squared-distance threshold that no improving candidate can exceed: an
// improving b has sqrt_rn(D2) <= W <= W*, hence D2 <= W*^2 (1 + 2^-23 + ...),
// below W*^2 (1 + 2^-20) even after the two roundings of this product.
__device__ __forceinline__ float scan_threshold(float w) {
    if (w < 1e-18f) return 1e-36f;
    const float t = w * w * 1.00000095367431640625f;
    return t < FLT_MAX ? t : FLT_MAX;
}

template <int CB, int RB> struct EpiScan {
    uint64_t best[CB];
    uint64_t init[CB];
    float thr[CB];
    float na[CB];
    float corea[CB];
    int32_t ca[CB];
    int g;

    __device__ __forceinline__ void candidate(int cb, float d2, int32_t j, int32_t cj, float corej) {
        if (cj == ca[cb]) return;
        const float D = sqrt_rn(d2 > 0.f ? d2 : 0.f);
        const float W = fmaxf(fmaxf(corea[cb], corej), D);
        const uint64_t key = ((uint64_t)__float_as_uint(W) << 32) | (uint32_t)j;
        if (key < best[cb]) {
            best[cb] = key;
            thr[cb] = scan_threshold(W);
        }
    }
    __device__ __forceinline__ void tile(const f4 (&acc)[RB][CB], const float *nrm, const int32_t *comp,
                                         const float *core, int64_t j0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const f4 nb4 = *reinterpret_cast<const f4 *>(nrm + rb * 16 + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rb * 16 + 4 * g + r;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const float d2 = fmaf(-2.f, acc[rb][cb][r], na[cb] + nb4[r]);
                    if (d2 <= thr[cb]) candidate(cb, d2, (int32_t)(j0 + row), comp[row], core[row]);
                }
            }
        }
    }
};

template <int QM> __global__ __launch_bounds__(kThreads) void scan_tile_kernel(ScanArgs a) {
    constexpr int CB = scan_col_blocks(QM);
    using T = Tile<QM, CB>;
    constexpr int QT = kWaves * 16 * CB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
    const int split = blockIdx.y;
    const int64_t cbase = (int64_t)blockIdx.x * QT;

    EpiScan<CB, T::RB> epi;
    epi.g = g;
    float bq[CB][QM];
    int32_t pt[CB];
    bool valid[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t c = cbase + wave * 16 * CB + cb * 16 + li;
        valid[cb] = c < a.nact;
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
        epi.thr[cb] = (!valid[cb] || epi.corea[cb] > w0) ? -INFINITY : scan_threshold(w0);
    }
    const int64_t tb = a.tiles * split / a.splits, te = a.tiles * (split + 1) / a.splits;
    run_tiles<QM, CB, true>(a.X, a.ldx, a.n, a.nrm, a.comp, a.core, a.d, a.chunks, tb, te, bq, epi);

#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        uint64_t b = epi.best[cb];
#pragma unroll
        for (int mask = 16; mask <= 32; mask <<= 1) {
            const uint32_t lo = __shfl_xor((uint32_t)b, mask), hi = __shfl_xor((uint32_t)(b >> 32), mask);
            const uint64_t o = ((uint64_t)hi << 32) | lo;
            b = o < b ? o : b;
        }
        if (g == 0 && valid[cb] && b < epi.init[cb]) atomicMin((unsigned long long *)&a.best[pt[cb]], (unsigned long long)b);
    }
}

template <int QM> static hipError_t scan_launch(const ScanArgs &a, hipStream_t s) {
    constexpr int QT = kWaves * 16 * scan_col_blocks(QM);
    const dim3 grid((unsigned)((a.nact + QT - 1) / QT), (unsigned)a.splits);
    hipLaunchKernelGGL(scan_tile_kernel<QM>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_scan_tile(int QM, const ScanArgs &a, hipStream_t s) {
    if (a.nact <= 0) return hipSuccess;
    switch (QM) {
    case 16: return scan_launch<16>(a, s);
    case 32: return scan_launch<32>(a, s);
    case 64: return scan_launch<64>(a, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace ekh
