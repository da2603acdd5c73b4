// Device templates shared by the dense tile kernels of libekh (gfx950).
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
#pragma once

#include "ekh_internal.h"

#include <float.h>
#include <math.h>

#include <type_traits>

namespace ekh {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma16(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- tile loop
// Feature order of the contraction: with QM = 2 * ceil(d / 8) k-steps, lane
// group g supplies feature g * QM + s at k-step s (features >= d are zero).
// Any fixed assignment of features to (s, g) gives the same dot product up to
// rounding; using this one in every kernel keeps D2 bitwise identical (and
// symmetric).  In a point-major row (and an LDS tile row) group g's features
// sit at positions g * QP + s, QP = QM rounded up to 4, so a lane reads four
// consecutive k-steps of its A operand with one aligned 16-byte LDS read.
template <int QM> struct Tile {
    static constexpr int TR = TileGeo<QM>::TR;  // database rows per tile
    static constexpr int RB = TR / 16;          // 16-row blocks per tile
    static constexpr int QP = qm_pad(QM);       // positions of a lane group's segment
    static constexpr int FD = QP * 4;           // floats per row (tile_dim(d))
    static constexpr int RS = FD + 4;           // LDS row stride in floats: 16-byte reads of 8 rows hit distinct banks
    static constexpr int NP = TR * QP;          // 16-byte pieces per tile
    static constexpr int NL = (NP + kThreads - 1) / kThreads; // pieces each thread loads per tile
};

// Streams database tiles [t_begin, t_end) through LDS tile buffers
// (row-major: [row][feature]) and hands each tile's accumulator blocks to
// epi.tile().  With TPB = 1, two buffers and one barrier per tile: the global
// loads of tile t + 1 are in flight while the MFMAs and the epilogue of tile t
// run.  With TPB = 2, four buffers and one barrier per two tiles (see the
// loop).  One
// accumulator set and one prefetch set keep the registers low enough for
// three waves per SIMD (d <= 64), so that while one wave waits at its barrier
// or works through its epilogue, the others keep the MFMA pipe busy.  Per-row
// norms (and, with PAYLOAD, component labels and core distances) live in a
// second set of LDS slots, tile t's in the slot of its features' buffer: a
// slot is refilled only after a barrier that follows its tile's epilogue.
// Each buffer's MFMA block and stores are separate code, so their LDS
// addresses are immediate offsets rather than per-tile vector additions.
// The kernels are instantiated per k-step count, so the k-loop runs all QM
// k-steps, fully unrolled, with the next k-steps' A operands read ahead.
//
// The database is read from its point-major copy Bp: row j holds point j in
// the segment layout above, dp = 4 * QP floats (zero at the padding
// positions and past d), so a tile is one contiguous block of TR * dp floats.  Thread tid loads its 16-byte
// pieces tid, tid + 256, ... of the block (coalesced) with buffer loads whose
// base is the tile's first row (a scalar) and whose lane offsets never change;
// each piece goes to LDS with one 16-byte store.  Point counts are below 2^31,
// so tile and row counters are 32-bit scalars.
template <int QM, int CB, bool PAYLOAD, int TPB, class Epi>
__device__ __forceinline__ void run_tiles(const float *__restrict__ Bp, int32_t m_, const float *__restrict__ nrm_b,
                                          const int32_t *__restrict__ comp_b, const float *__restrict__ core_b,
                                          int32_t t_begin_, int32_t t_end_, const float (&bq)[CB][QM], Epi &epi) {
    using T = Tile<QM>;
    const uint32_t t_begin = __builtin_amdgcn_readfirstlane((uint32_t)t_begin_);
    const uint32_t t_end = __builtin_amdgcn_readfirstlane((uint32_t)t_end_);
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)m_);
    constexpr int NBUF = 2 * TPB;
    __shared__ __align__(16) float sm_tile[NBUF][T::TR * T::RS];
    __shared__ __align__(16) float sm_nrm[NBUF][T::TR];
    __shared__ int32_t sm_comp[NBUF][PAYLOAD ? T::TR : 1];
    __shared__ float sm_core[NBUF][PAYLOAD ? T::TR : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, li = lane & 15;

    // this thread's pieces: LDS position (row * RS + 4 * column) and whether
    // the piece exists (a tile may have fewer pieces than 256 * NL)
    int lds_off[T::NL];
    bool has[T::NL];
#pragma unroll
    for (int h = 0; h < T::NL; ++h) {
        const int c = tid + kThreads * h;
        has[h] = T::NP % kThreads == 0 || c < T::NP;
        const int row = c / T::QP, col = c - row * T::QP;
        lds_off[h] = row * T::RS + 4 * col;
    }
    const int lrow = tid % T::TR; // the thread also loads row lrow's norm (and payload)
    // in a database of fewer rows than one tile, the lanes past its end read
    // row m - 1 instead (with an infinite norm)
    const uint32_t lr = m < (uint32_t)T::TR && (uint32_t)lrow >= m ? m - 1 : (uint32_t)lrow;

    struct Pref {
        f4 v[T::NL];
        float n, core;
        int32_t comp;
        bool nv;       // a row of this tile (else an infinite norm)
        uint32_t row0; // first row read
    };
    typedef const char __attribute__((address_space(1))) *gchar;
    auto sbase = [](const void *ptr) {
        const uint64_t x = reinterpret_cast<uint64_t>(ptr);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
        return (gchar)(((uint64_t)hi << 32) | lo);
    };
    // raw buffer loads from a scalar base; bytes past `bytes` read as zero
    auto rsrc = [](gchar base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)(const char *)base, (short)0, (int)bytes, 0x00020000);
    };
    constexpr uint32_t row_bytes = (uint32_t)T::FD * 4u;
    const bool short_db = m < (uint32_t)T::TR;                              // the database is shorter than a tile
    const uint32_t last0 = __builtin_amdgcn_readfirstlane(short_db ? 0u : m - T::TR); // first row of a partial last tile
    // One load sequence for every tile, with no address arithmetic (a branch
    // around the loads would cost the wait counts that let the next tile's
    // loads overlap this tile's MFMAs).  A partial last tile is read as rows
    // m - TR .. m - 1 (a change of base); its rows before the tile belong to
    // the previous one and get an infinite norm, so they never qualify.
    auto load = [&](Pref &P, uint32_t t) {
        const uint32_t tt = t < t_end ? t : t_end - 1;
        const uint32_t rt = tt * (uint32_t)T::TR; // the tile's first row (< 2^32: m < 2^31)
        const bool part = rt + (uint32_t)T::TR > m;
        const uint32_t row0 = part ? last0 : rt;
        P.row0 = row0;
        // rows lrow in [lo, hi) belong to this tile (scalar bounds)
        const uint32_t lo = part && !short_db ? rt - row0 : 0u;
        const uint32_t hi = part && short_db ? m : (uint32_t)T::TR;
        P.nv = (uint32_t)lrow >= lo && (uint32_t)lrow < hi;
        const uint32_t rows = m - row0 < (uint32_t)T::TR ? m - row0 : (uint32_t)T::TR;
        const auto r = rsrc(sbase(Bp + (uint64_t)row0 * (uint32_t)T::FD), rows * row_bytes);
        // pieces past the tile (more threads than pieces, or rows past m) lie
        // past the resource's end: they read as zeros and are not stored
#pragma unroll
        for (int h = 0; h < T::NL; ++h) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (tid + kThreads * h) * 16, 0, 0);
            P.v[h] = f4{__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3])};
        }
        const auto rn = rsrc(sbase(nrm_b + row0), 0x7fffffff);
        P.n = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rn, lr * 4u, 0, 0));
        if (PAYLOAD) {
            P.comp = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc(sbase(comp_b + row0), 0x7fffffff), lr * 4u, 0, 0);
            P.core = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rsrc(sbase(core_b + row0), 0x7fffffff), lr * 4u, 0, 0));
        }
    };
    auto store = [&](const Pref &P, auto BUF) {
        constexpr int buf = decltype(BUF)::value;
#pragma unroll
        for (int h = 0; h < T::NL; ++h)
            if (has[h]) *reinterpret_cast<f4 *>(sm_tile[buf] + lds_off[h]) = P.v[h];
        if (tid < T::TR) {
            sm_nrm[buf][tid] = P.nv ? P.n : INFINITY; // padding rows never qualify
            if (PAYLOAD) {
                sm_comp[buf][tid] = P.nv ? P.comp : -1;
                sm_core[buf][tid] = P.nv ? P.core : INFINITY;
            }
        }
    };
    auto mma = [&](auto BUF, f4 (&acc)[T::RB][CB]) {
        constexpr int buf = decltype(BUF)::value;
#pragma unroll
        for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f4{0.f, 0.f, 0.f, 0.f};
        // this lane's feature segment of each row it reads
        const float *tl = sm_tile[buf] + li * T::RS + g * T::QP;
        constexpr int PRE = 4; // k-steps whose A operands are read at once (one 16-byte read per row block)
#pragma unroll
        for (int s0 = 0; s0 < QM; s0 += PRE) {
            f4 a4[T::RB];
#pragma unroll
            for (int rb = 0; rb < T::RB; ++rb) a4[rb] = *reinterpret_cast<const f4 *>(tl + rb * 16 * T::RS + s0);
#pragma unroll
            for (int s = 0; s < PRE && s0 + s < QM; ++s)
#pragma unroll
                for (int rb = 0; rb < T::RB; ++rb)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mfma16(a4[rb][s], bq[cb][s0 + s], acc[rb][cb]);
        }
    };
    auto finish = [&](const f4 (&acc)[T::RB][CB], uint32_t row0, int slot) {
        epi.tile(acc, sm_nrm[slot], PAYLOAD ? sm_comp[slot] : nullptr, PAYLOAD ? sm_core[slot] : nullptr,
                 (int64_t)row0);
    };

    if (t_begin >= t_end) return;
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    Pref P;
    f4 acc[T::RB][CB];
    if constexpr (TPB == 1) {
        load(P, t_begin);
        store(P, B0{});
        __syncthreads();
        uint32_t rcur = P.row0; // tile t's first row
        for (uint32_t t = t_begin; t < t_end; ++t) {
            const bool odd = ((t - t_begin) & 1u) != 0u; // wave-uniform: tile t's buffer and norm slot
            if (t + 1 < t_end) load(P, t + 1);
            if (odd)
                mma(B1{}, acc);
            else
                mma(B0{}, acc);
            finish(acc, rcur, odd ? 1 : 0);
            if (t + 1 < t_end) {
                if (odd)
                    store(P, B0{});
                else
                    store(P, B1{});
            }
            __syncthreads();
            rcur = P.row0;
        }
    } else {
        // Four buffers, tile t in buffer (t - t_begin) mod 4, and a barrier after
        // every second tile: tile t + 2 is loaded while tile t's MFMAs and
        // epilogue run and stored into the buffer that tile t - 2 used (read
        // before the barrier that followed tile t - 1 or t - 2), and a barrier
        // separates that store from tile t + 2's reads.
        static_assert(TPB == 2, "one or two tiles per barrier");
        using B2 = std::integral_constant<int, 2>;
        using B3 = std::integral_constant<int, 3>;
        load(P, t_begin);
        store(P, B0{});
        uint32_t r0 = P.row0, r1 = P.row0; // first rows of tiles t and t + 1
        if (t_begin + 1 < t_end) {
            load(P, t_begin + 1);
            store(P, B1{});
            r1 = P.row0;
        }
        __syncthreads();
        for (uint32_t t = t_begin; t < t_end; ++t) {
            const uint32_t b = (t - t_begin) & 3u; // wave-uniform: tile t's buffer and norm slot
            const bool next = t + 2 < t_end;
            if (next) load(P, t + 2);
            switch (b) {
            case 0: mma(B0{}, acc); break;
            case 1: mma(B1{}, acc); break;
            case 2: mma(B2{}, acc); break;
            default: mma(B3{}, acc); break;
            }
            finish(acc, r0, (int)b);
            if (next) {
                switch (b) {
                case 0: store(P, B2{}); break;
                case 1: store(P, B3{}); break;
                case 2: store(P, B0{}); break;
                default: store(P, B1{}); break;
                }
            }
            if (b & 1u) __syncthreads();
            r0 = r1;
            r1 = P.row0;
        }
    }
}

// Loads the register-resident query operand: lane (g, i) holds feature
// g * QM + s of its query column at k-step s.
template <int QM>
__device__ __forceinline__ void load_query(const float *__restrict__ Q, int64_t ldq, int64_t col, bool valid, int d,
                                           int g, float (&bq)[QM]) {
#pragma unroll
    for (int s = 0; s < QM; ++s) {
        const int f = g * QM + s;
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
    // Candidate from a stream whose indices ascend (v < d[K - 1] required): it is
    // larger than every entry in index, so a strict '<' on d2 keeps equal
    // distances in index order.  The new list is a fixed network with no serial
    // chain: slot t takes the median of (old t - 1, v, old t), which is old t
    // before v's place, v at it and old t - 1 after it; the indices follow the
    // same two comparisons.  Same result as moving v down by compare-and-swaps.
    __device__ __forceinline__ void push_ascending(float v, int32_t j) {
        bool lt[K];
#pragma unroll
        for (int t = 0; t < K; ++t) lt[t] = v < d[t];
        float nd[K];
        int32_t ni[K];
        nd[0] = lt[0] ? v : d[0];
        ni[0] = lt[0] ? j : i[0];
#pragma unroll
        for (int t = 1; t < K; ++t) {
            nd[t] = __builtin_amdgcn_fmed3f(d[t - 1], v, d[t]);
            ni[t] = lt[t - 1] ? i[t - 1] : (lt[t] ? j : i[t]);
        }
#pragma unroll
        for (int t = 0; t < K; ++t) {
            d[t] = nd[t];
            i[t] = ni[t];
        }
    }
    // (d2, idx) order as one 64-bit comparison: for d2 >= 0 (or +inf) the float
    // bits order like the values, and indices are non-negative.
    __device__ __forceinline__ static uint64_t key(float a, int32_t ia) {
        return ((uint64_t)__float_as_uint(a) << 32) | (uint32_t)ia;
    }
    __device__ __forceinline__ static bool less(float a, int32_t ia, float b, int32_t ib) {
        return key(a, ia) < key(b, ib);
    }
    // Candidate in any order: the same fixed network as push_ascending, with the
    // full (d2, idx) comparison deciding where the candidate goes.  med3 still
    // yields the right value in every slot (where the candidate ties a
    // neighbour on d2, either choice is the same value); the indices follow the
    // full comparisons.  No serial chain, so the K slots update in parallel.
    __device__ __forceinline__ void push_any(float v, int32_t j) {
        bool lt[K];
#pragma unroll
        for (int t = 0; t < K; ++t) lt[t] = less(v, j, d[t], i[t]);
        float nd[K];
        int32_t ni[K];
        nd[0] = lt[0] ? v : d[0];
        ni[0] = lt[0] ? j : i[0];
#pragma unroll
        for (int t = 1; t < K; ++t) {
            nd[t] = __builtin_amdgcn_fmed3f(d[t - 1], v, d[t]);
            ni[t] = lt[t - 1] ? i[t - 1] : (lt[t] ? j : i[t]);
        }
#pragma unroll
        for (int t = 0; t < K; ++t) {
            d[t] = nd[t];
            i[t] = ni[t];
        }
    }
    // Whether (v, j) would enter the list.
    __device__ __forceinline__ bool admits(float v, int32_t j) const { return less(v, j, d[K - 1], i[K - 1]); }
    // Pushes a list that ascends in (d2, idx): once no lane of the wave admits
    // its next entry, no later entry can enter either (each lane's last entry
    // only falls), so the wave stops there.
    __device__ __forceinline__ void push_sorted(const float (&od)[K], const int32_t (&oi)[K]) {
#pragma unroll
        for (int t = 0; t < K; ++t) {
            if (!__builtin_amdgcn_ballot_w64(admits(od[t], oi[t]))) break;
            push_any(od[t], oi[t]);
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
        push_sorted(od, oi);
    }
};

// The K smallest values only (no indices): the bound pass of the symmetric
// self-kNN needs the K-th smallest D2 of each row, a value, which any choice
// among equal values leaves the same.  Insertion: slot t takes med3(old t - 1,
// v, old t), slot 0 min(v, old 0); no comparison, no index to carry.
template <int K> struct TopV {
    float d[K];

    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int t = 0; t < K; ++t) d[t] = INFINITY;
    }
    __device__ __forceinline__ void push(float v) {
        float nd[K];
        nd[0] = fminf(v, d[0]);
#pragma unroll
        for (int t = 1; t < K; ++t) nd[t] = __builtin_amdgcn_fmed3f(d[t - 1], v, d[t]);
#pragma unroll
        for (int t = 0; t < K; ++t) d[t] = nd[t];
    }
    __device__ __forceinline__ void push_ascending(float v, int32_t) { push(v); }
    // pushes an ascending list; stops once no lane of the wave has a value below its last
    __device__ __forceinline__ void push_sorted(const float (&od)[K]) {
#pragma unroll
        for (int t = 0; t < K; ++t) {
            if (!__builtin_amdgcn_ballot_w64(od[t] < d[K - 1])) break;
            push(od[t]);
        }
    }
    __device__ __forceinline__ void merge_xor(int mask) {
        float od[K];
#pragma unroll
        for (int t = 0; t < K; ++t) od[t] = __shfl_xor(d[t], mask);
        push_sorted(od);
    }
};

// ---------------------------------------------------------------- lane groups
// Min / max over the four lanes (lane ^ 16, lane ^ 32) that share a query
// column, with the gfx950 lane-swap instructions: permlane16_swap(v, v) yields
// v and the value of lane ^ 16 (in an order that depends on the row), and
// permlane32_swap likewise for lane ^ 32, so a symmetric min or max needs no
// lane select and no LDS round trip.
__device__ __forceinline__ uint32_t group_min_u32(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const uint32_t m = a[0] < a[1] ? a[0] : a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return b[0] < b[1] ? b[0] : b[1];
}
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const uint32_t m = a[0] > a[1] ? a[0] : a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return b[0] > b[1] ? b[0] : b[1];
}
// Second largest of the eight values (a_g, b_g), a_g >= b_g, held by the four
// lanes of a column: merge (largest, second largest) pairs across lane ^ 16 and
// lane ^ 32.  The merge of (x1, x2) and (y1, y2) is (max(x1, y1),
// max(min(x1, y1), x2, y2)), symmetric, so the swap order does not matter.
__device__ __forceinline__ uint32_t group_second_u32(uint32_t a, uint32_t b) {
    auto pa = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    auto pb = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    uint32_t t1 = pa[0] > pa[1] ? pa[0] : pa[1];
    uint32_t t2 = pa[0] < pa[1] ? pa[0] : pa[1];
    uint32_t b2 = pb[0] > pb[1] ? pb[0] : pb[1];
    t2 = t2 > b2 ? t2 : b2;
    pa = __builtin_amdgcn_permlane32_swap(t1, t1, false, false);
    pb = __builtin_amdgcn_permlane32_swap(t2, t2, false, false);
    const uint32_t m = pa[0] < pa[1] ? pa[0] : pa[1];
    b2 = pb[0] > pb[1] ? pb[0] : pb[1];
    return m > b2 ? m : b2;
}
// For non-negative floats (and +inf) the bit patterns order like the values.
__device__ __forceinline__ float group_min_nonneg(float v) { return __uint_as_float(group_min_u32(__float_as_uint(v))); }
__device__ __forceinline__ float group_max_nonneg(float v) { return __uint_as_float(group_max_u32(__float_as_uint(v))); }

// ---------------------------------------------------------------- kNN epilogue
// Each lane keeps CB lists (one per query column it owns) in registers.  Per
// tile every D2 is tested against an admission threshold in straight-line code
// (the fast test); only when a lane of the wave passes, the slow path inserts
// the passing rows of each lane in ascending row order (see slow()).
//
// The four lanes of a query column see disjoint rows and keep separate lists
// that are merged at the end.  Any K real candidates bound the query's final
// K-th D2 from above, and two such bounds are cheap to share between the four
// lanes: the smallest of their last entries (one full list), and the K-th
// smallest of their first J + 1 entries, J = ceil(K / 4) - 1 (four lists with
// J + 1 entries each hold at least K candidates).  That is the largest of the
// four J-th entries, or, when 4 (J + 1) = K + 1 (K = 11), the second largest of
// the eight J-th and (J - 1)-th entries.  A candidate above the smaller bound can never
// reach the final list and is not admitted (on equality it is, since a lower
// index can still win the tie).  Without this, each lane would keep filling its
// own list with candidates that the final merge drops.
template <int K, int CB, int RB, class List = TopK<K>> struct EpiKnn {
    static constexpr int J = (K + 3) / 4 - 1;
    static constexpr bool kSecond = 4 * (J + 1) == K + 1 && J >= 1;
    List lst[CB]; // this lane's lists, in registers
    float nq[CB];
    float admq[CB]; // admission bound on D2 shared by the column's four lanes, moved to nb - 2 s and widened
                    // by the rounding margin
    bool dirty[CB]; // wave-uniform: a lane of the wave inserted into list cb since its bound was last formed
    int32_t qrow[CB];
    int g;

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            lst[cb].clear();
            admq[cb] = INFINITY;
            dirty[cb] = false;
        }
    }
    __device__ __forceinline__ void load(int cb, List &L) { L = lst[cb]; }
    __device__ __forceinline__ void store(int cb, const List &L) { lst[cb] = L; }

    // D2 = fma(-2, s, nq + nb).  The pair (i, i) needs no special case: the
    // norms come from the same MFMA chain as the dot products, so it is
    // fma(-2, n_i, 2 n_i) = 0 exactly.
    //
    // Fast test per element: t = fma(-2, s, nb) against admq = adm - nq, widened.
    // If D2 = fma(-2, s, nq + nb) (two roundings) is <= adm, the point lies within
    // sqrt(adm) of the query, so nb <= 2 nq + 2 adm, and every rounding error
    // between D2 and t + nq is at most a few units of 2^-24 (nq + nb + adm); the
    // widening by 2^-20 (adm + nq) covers it with room to spare.  The test only
    // decides which rows a lane inserts (with their exact D2): the margin can
    // admit a few more rows, which does not change the result (see slow()).
    //
    // prepare() re-forms the bound of each list block a lane of the wave
    // inserted into (a wave-uniform test per block), fast() is the branch-free
    // test, slow() inserts the candidates of the columns that passed; tile()
    // runs the three.  The bound comes from the lists' last, J-th and
    // (J - 1)-th entries.
    __device__ __forceinline__ void prepare() {
        constexpr float kWiden = 1.0f / 1048576.0f;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (dirty[cb]) {
                const List &L = lst[cb];
                const float gq = kSecond ? __uint_as_float(group_second_u32(__float_as_uint(L.d[J]),
                                                                             __float_as_uint(L.d[J - 1])))
                                         : group_max_nonneg(L.d[J]);
                const float adm = fminf(group_min_nonneg(L.d[K - 1]), gq);
                admq[cb] = fmaf(adm, 1.0f + kWiden, -nq[cb] * (1.0f - kWiden));
                dirty[cb] = false;
            }
        }
    }
    __device__ __forceinline__ void fast(const f4 (&acc)[RB][CB], const f4 (&nb4)[RB], bool (&hit)[CB]) const {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            float mn = INFINITY;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mn = fminf(mn, fmaf(-2.f, acc[rb][cb][r], nb4[rb][r]));
            hit[cb] = mn <= admq[cb];
        }
    }
    // Candidates of the lanes that passed, inserted in a loop over the set bits
    // of a per-lane mask (bit 4 rb + r: ascending rows).  Each trip, every lane
    // with a bit left takes its lowest, reads that row's dot product back from
    // LDS ([value][thread], so the row is picked by an address rather than a
    // chain of selects) and inserts the exact D2.  The fixed insertion network
    // thus runs as many times as the busiest lane of the wave has candidates,
    // not once per row position that any lane needs.
    //
    // The mask takes the fast test's value per row (t = fma(-2, s, n_b) against
    // the widened bound), a superset of the rows within the bound.  A row
    // beyond the bound that enters a list is still a real candidate of the
    // query, and the merged result stays exact: every row of the final list is
    // within the bound at every moment (the bound is the K-th smallest of K real
    // candidates, never below the final K-th), so no lane drops it, whatever
    // else its list holds.
    static constexpr int NV = CB * RB * 4;
    float *sv;  // LDS [NV][kThreads]
    int tid;
    __device__ __forceinline__ void slow(const f4 (&acc)[RB][CB], const f4 (&nb4)[RB], const bool (&hit)[CB],
                                         const float *nrm, int64_t j0) {
        bool any = false;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) any = any || hit[cb];
        if (!__builtin_amdgcn_ballot_w64(any)) return;
        stash(acc);
        insert(nb4, hit, acc, nrm, j0, [&](int cb, int e) {
            return sv[((cb * RB + (e >> 2)) * 4 + (e & 3)) * kThreads + tid];
        });
        __builtin_amdgcn_wave_barrier(); // the loads above before the next tile's stores
    }
    // the wave's dot products to LDS ([value][thread])
    __device__ __forceinline__ void stash(const f4 (&acc)[RB][CB]) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) sv[((cb * RB + rb) * 4 + r) * kThreads + tid] = acc[rb][cb][r];
        __builtin_amdgcn_wave_barrier(); // the LDS stores above before the loads below
    }
    // the insertions; dot(cb, e) gives the dot product of element e (= 4 rb + r) of block cb
    template <class Dot>
    __device__ __forceinline__ void insert(const f4 (&nb4)[RB], const bool (&hit)[CB], const f4 (&acc)[RB][CB],
                                           const float *nrm, int64_t j0, Dot dot) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (!__builtin_amdgcn_ballot_w64(hit[cb])) continue;
            dirty[cb] = true; // wave-uniform: this block's bound is re-formed before the next tile
            uint32_t mk = 0u;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mk |= fmaf(-2.f, acc[rb][cb][r], nb4[rb][r]) <= admq[cb] ? (1u << (4 * rb + r)) : 0u;
            List L;
            load(cb, L);
            for (int trip = 0; trip < RB * 4; ++trip) {
                if (!__builtin_amdgcn_ballot_w64(mk != 0u)) break;
                if (mk != 0u) {
                    const int e = __builtin_ctz(mk);
                    mk &= mk - 1u;
                    const int row = (e >> 2) * 16 + 4 * g + (e & 3);
                    const float d2 = fmaf(-2.f, dot(cb, e), nq[cb] + nrm[row]);
                    L.push_ascending(d2 > 0.f ? d2 : 0.f, (int32_t)(j0 + row));
                }
            }
            store(cb, L);
        }
    }
    __device__ __forceinline__ void tile(const f4 (&acc)[RB][CB], const float *nrm, const int32_t *, const float *,
                                         int64_t j0) {
        f4 nb4[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) nb4[rb] = *reinterpret_cast<const f4 *>(nrm + rb * 16 + 4 * g);
        prepare();
        bool hit[CB];
        fast(acc, nb4, hit);
        slow(acc, nb4, hit, nrm, j0);
    }
};

// A finished value list (the bound pass): its k_out-th value to out_core, or
// to the split scratch (index 0 for every entry: the merge keeps the values).
template <int K>
__device__ __forceinline__ void write_list(const KnnArgs &a, const TopV<K> &L, int64_t q, Entry *dst) {
    if (dst) {
#pragma unroll
        for (int t = 0; t < K; ++t) dst[t] = Entry{L.d[t], 0};
    } else {
        float c = 0.f;
#pragma unroll
        for (int t = 0; t < K; ++t)
            if (t == a.k_out - 1) c = L.d[t]; // a select per entry (no dynamic register index)
        a.out_core[q] = c;
    }
}

// Writes a finished list for absolute row q: to the split scratch at dst when
// it is one split's partial list, else in the final form a.out_mode names.
template <int K>
__device__ __forceinline__ void write_list(const KnnArgs &a, const TopK<K> &L, int64_t q, Entry *dst) {
    if (dst) {
#pragma unroll
        for (int t = 0; t < K; ++t) dst[t] = Entry{L.d[t], L.i[t]};
    } else if (a.out_mode == kOutBound) {
        float c = 0.f;
#pragma unroll
        for (int t = 0; t < K; ++t)
            if (t == a.k_out - 1) c = L.d[t]; // a select per entry (no dynamic register index)
        a.out_core[q] = c;
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

// VAL: value lists (the bound pass of the symmetric self-kNN, a.out_mode == kOutBound).  Without the
// indices the kernel fits 128 VGPRs, so it runs four waves per SIMD with one barrier per tile (two LDS
// tile buffers: four workgroups per CU)
template <int K, int QM, bool VAL = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(VAL ? 4 : knn_waves_per_simd(K, QM),
                                                                           VAL ? 4 : knn_waves_per_simd(K, QM))))
void knn_tile_kernel(KnnArgs a) {
    using List = typename std::conditional<VAL, TopV<K>, TopK<K>>::type;
    constexpr int CB = knn_col_blocks(K, QM);
    using T = Tile<QM>;
    constexpr int QT = kWaves * 16 * CB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
    // one-dimensional grid: the first body_q query tiles each take the whole
    // database in one workgroup, then every remaining query tile takes one
    // workgroup per database split (split-major order)
    const int64_t tail0 = a.body_q * QT;              // local row of the first split tile
    const int64_t tail_q = (a.nq - tail0 + QT - 1) / QT;
    const bool body = (int64_t)blockIdx.x < a.body_q;
    const int64_t h = body ? 0 : (int64_t)blockIdx.x - a.body_q;
    const int split = body ? 0 : (int)(h / tail_q);
    const int nsplit = body ? 1 : a.splits;
    const int64_t qbase = body ? (int64_t)blockIdx.x * QT : tail0 + (h % tail_q) * QT; // local row of the first query
    if (a.gate && a.gate[(a.q0 + qbase) / a.gate_rows] == 0u) return; // a tile that need not run

    float bq[CB][QM];
    bool qv[CB];
    float nq[CB];
    int32_t qrow[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t ql = qbase + wave * 16 * CB + cb * 16 + li;
        qv[cb] = ql < a.nq;
        const int64_t q = a.q0 + (qv[cb] ? ql : 0);
        load_query<QM>(a.Q, a.ldq, q, qv[cb], a.d, g, bq[cb]);
        nq[cb] = qv[cb] ? a.nrm_q[q] : 0.f;
        qrow[cb] = (int32_t)(a.q0 + ql);
    }
    const int64_t tb = a.tiles * split / nsplit, te = a.tiles * (split + 1) / nsplit;

    __shared__ float sv[EpiKnn<K, CB, T::RB, List>::NV * kThreads];
    EpiKnn<K, CB, T::RB, List> epi;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        epi.nq[cb] = nq[cb];
        epi.qrow[cb] = qrow[cb];
    }
    epi.init();
    epi.g = g;
    epi.sv = sv;
    epi.tid = tid;
    run_tiles<QM, CB, false, VAL ? 1 : knn_tiles_per_barrier(QM)>(a.Bt, (int32_t)a.m, a.nrm_b, nullptr, nullptr, (int32_t)tb, (int32_t)te, bq, epi);

    // merge the four lane groups that share each query column
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        List L;
        epi.load(cb, L);
        L.merge_xor(16);
        L.merge_xor(32);
        Entry *dst = nullptr;
        if (nsplit > 1) dst = a.part + ((int64_t)split * (a.nq - tail0) + (epi.qrow[cb] - a.q0 - tail0)) * K;
        if (g == 0 && qv[cb]) write_list<K>(a, L, epi.qrow[cb], dst);
    }
}

// Split lists of the split tiles' rows (a.q0, a.nq name them), merged by
// kMergeLanes lanes per row: lane r takes splits r, r + kMergeLanes, ..., then
// the lanes' lists are combined by xor merges (full (D2, index) comparisons on
// disjoint sets, so any order gives the same list).
constexpr int kMergeLanes = 16;
static_assert(64 % kMergeLanes == 0, "a row's lanes lie in one wave");
template <int K> __global__ __launch_bounds__(256) void knn_merge_kernel(KnnArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ql = gid / kMergeLanes;
    const int r = (int)(gid % kMergeLanes);
    TopK<K> L;
    L.clear();
    // rows of query tiles that did not run (a.gate) are skipped like rows past the end
    const bool row = ql < a.nq && (!a.gate || a.gate[(a.q0 + ql) / a.gate_rows] != 0u);
    // the lanes of a wave run the same number of trips (a.splits is uniform and
    // r < kMergeLanes): lanes past their last split push empty lists
    for (int s0 = 0; s0 < a.splits; s0 += kMergeLanes) {
        const int s = s0 + r;
        float od[K];
        int32_t oi[K];
        const bool have = row && s < a.splits;
        const Entry *src = a.part + ((int64_t)(have ? s : 0) * a.nq + (have ? ql : 0)) * K;
#pragma unroll
        for (int t = 0; t < K; ++t) {
            const Entry e = have ? src[t] : Entry{INFINITY, 0x7fffffff};
            od[t] = e.d2;
            oi[t] = e.idx;
        }
        L.push_sorted(od, oi);
    }
    // every lane of the wave takes part in the shuffles (rows past the end hold empty lists)
#pragma unroll
    for (int mask = 1; mask < kMergeLanes; mask <<= 1) L.merge_xor(mask);
    if (row && r == 0) write_list<K>(a, L, a.q0 + ql, 0);
}

// ---------------------------------------------------------------- symmetric self-kNN
// D2 is bitwise symmetric (the same chain of products in the same k-order for
// (i, j) and (j, i)), so the self-kNN computes every pair once: query tile t
// (QT points, rows [t QT, (t + 1) QT)) runs over the database rows from its own
// first row on, the upper block triangle.  A pair (i, j) it computes feeds
// i's list (the row side, as in knn_tile_kernel) and, when j lies past the
// query tile's own block, j's list through a candidate buffer (the column
// side).  Every pair of points is then seen by both of its lists: within a
// block by the row side, across blocks by the row side of the earlier block
// and the column side of the later one.
//
// Both sides admit a candidate only within a bound on its point's final
// k-th D2: tau, the k-th D2 among a subset of the points (a bound, since those
// are real candidates).  The row side starts with tau instead of an empty
// list's infinite bound (no warm-up); the column side appends (D2, i) to j's
// buffer when D2 <= tau_j, so no candidate of the final list is missed.
// sym_merge_kernel merges the row side's lists with the buffer; a buffer
// that overflowed marks its query tile, whose lists the ordinary kernel then
// recomputes (a.gate).
//
// Column side's fast test per element, with t = fma(-2, s, n_j) from the row
// side: u = t - theta_j against -n_i, theta_j = tau_j + 2^-19 (n_j + tau_j).
// For D2 = fma(-2, s, n_i + n_j) <= tau_j the point i lies within sqrt(tau_j)
// of j, so n_i <= 2 n_j + 2 tau_j, and D2 and t + n_i differ by at most a few
// units of 2^-24 (n_i + n_j + tau_j) < 2^-21 (n_j + tau_j); theta_j's widening
// covers that and theta_j's own rounding, and the rounding of t - theta_j
// keeps the order.  The exact D2 decides (the same value the row side uses).
template <int K, int CB, int RB> struct EpiSym : EpiKnn<K, CB, RB> {
    using Base = EpiKnn<K, CB, RB>;
    float cap[CB];      // the query's bound tau (-inf for a column past the points)
    bool qv[CB];        // the query column holds a point
    int64_t col_from;   // database rows >= col_from take the column side (past the query tile's block)
    Entry *colbuf;
    uint32_t *colcnt;
    int colcap;
    // The slow paths take each passing element's dot product from registers (a
    // select over the lane's RB * 4 values) and append column candidates to the
    // buffers directly (a returning atomicAdd on the row's count, then a store):
    // no LDS stash and no LDS queue, so a workgroup needs only the tile loop's
    // LDS and fits five per CU.
    __device__ __forceinline__ static float dot_of(const f4 (&acc)[RB][CB], int cb, int e) {
        float v = acc[0][cb][0];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (rb * 4 + r > 0) v = e == rb * 4 + r ? acc[rb][cb][r] : v;
        return v;
    }

    // Base::prepare with the bound capped by tau
    __device__ __forceinline__ void prepare() {
        constexpr float kWiden = 1.0f / 1048576.0f;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (this->dirty[cb]) {
                const TopK<K> &L = this->lst[cb];
                const float gq = Base::kSecond ? __uint_as_float(group_second_u32(
                                                     __float_as_uint(L.d[Base::J]), __float_as_uint(L.d[Base::J - 1])))
                                               : group_max_nonneg(L.d[Base::J]);
                const float adm = fminf(fminf(group_min_nonneg(L.d[K - 1]), gq), cap[cb]);
                this->admq[cb] = fmaf(adm, 1.0f + kWiden, -this->nq[cb] * (1.0f - kWiden));
                this->dirty[cb] = false;
            }
        }
    }
    // comp: the rows' tau (bits), core: their theta (tile payload)
    __device__ __forceinline__ void tile(const f4 (&acc)[RB][CB], const float *nrm, const int32_t *tau_bits,
                                         const float *theta, int64_t j0) {
        const int g = this->g;
        f4 nb4[RB], th4[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            nb4[rb] = *reinterpret_cast<const f4 *>(nrm + rb * 16 + 4 * g);
            th4[rb] = *reinterpret_cast<const f4 *>(theta + rb * 16 + 4 * g);
        }
        prepare();
        // wave-uniform: a row of this tile lies past the query tile's block
        const bool colside = j0 + RB * 16 > col_from;
        bool hit[CB], hitc[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            float mn = INFINITY, mc = INFINITY;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float t = fmaf(-2.f, acc[rb][cb][r], nb4[rb][r]);
                    mn = fminf(mn, t);
                    mc = fminf(mc, t - th4[rb][r]);
                }
            hit[cb] = mn <= this->admq[cb];
            hitc[cb] = colside && mc <= -this->nq[cb];
        }
        bool anyr = false, anyc = false;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            anyr = anyr || hit[cb];
            anyc = anyc || hitc[cb];
        }
        const bool wr = __builtin_amdgcn_ballot_w64(anyr) != 0, wc = __builtin_amdgcn_ballot_w64(anyc) != 0;
        if (!wr && !wc) return;
        if (wc) column(acc, nb4, th4, hitc, tau_bits, nrm, j0);
        if (wr) this->insert(nb4, hit, acc, nrm, j0, [&](int cb, int e) { return dot_of(acc, cb, e); });
    }
    // Column side's candidates: a loop over the set bits of a per-lane mask as
    // in the row side, each appending the exact D2 to the database row's buffer
    // when it is within the row's tau.
    __device__ __forceinline__ void column(const f4 (&acc)[RB][CB], const f4 (&nb4)[RB], const f4 (&th4)[RB],
                                           const bool (&hitc)[CB], const int32_t *tau_bits, const float *nrm,
                                           int64_t j0) {
        const int g = this->g;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            if (!__builtin_amdgcn_ballot_w64(hitc[cb])) continue;
            uint32_t mk = 0u;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mk |= fmaf(-2.f, acc[rb][cb][r], nb4[rb][r]) - th4[rb][r] <= -this->nq[cb] ? (1u << (4 * rb + r))
                                                                                                 : 0u;
            if (!qv[cb]) mk = 0u;
            for (int trip = 0; trip < RB * 4; ++trip) {
                if (!__builtin_amdgcn_ballot_w64(mk != 0u)) break;
                bool take = false;
                float d2 = 0.f;
                int32_t j = 0;
                if (mk != 0u) {
                    const int e = __builtin_ctz(mk);
                    mk &= mk - 1u;
                    const int row = (e >> 2) * 16 + 4 * g + (e & 3);
                    j = (int32_t)(j0 + row);
                    d2 = fmaf(-2.f, dot_of(acc, cb, e), this->nq[cb] + nrm[row]);
                    d2 = d2 > 0.f ? d2 : 0.f;
                    // rows outside the tile carry NaN bits here, which no D2 satisfies
                    take = j0 + row >= col_from && d2 <= __int_as_float(tau_bits[row]);
                }
                if (take) {
                    const uint32_t pos = atomicAdd(&colcnt[j], 1u);
                    if (pos < (uint32_t)colcap) colbuf[(int64_t)j * colcap + pos] = Entry{d2, this->qrow[cb]};
                }
            }
        }
    }
};

template <int K, int QM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sym_waves_per_simd(K, QM), sym_waves_per_simd(K, QM))))
void knn_sym_kernel(KnnArgs a) {
    constexpr int CB = sym_col_blocks(K, QM);
    using T = Tile<QM>;
    constexpr int QT = kWaves * 16 * CB;
    static_assert(QT % T::TR == 0, "a query tile covers whole database tiles");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
    // item = query tile x split (query tiles in order, the longest ranges first)
    const int64_t qt = (int64_t)blockIdx.x / a.splits;
    const int split = (int)((int64_t)blockIdx.x % a.splits);
    const int64_t qbase = qt * QT;

    float bq[CB][QM];
    EpiSym<K, CB, T::RB> epi;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t q = qbase + wave * 16 * CB + cb * 16 + li;
        epi.qv[cb] = q < a.nq;
        const int64_t qs = epi.qv[cb] ? q : 0;
        load_query<QM>(a.Q, a.ldq, qs, epi.qv[cb], a.d, g, bq[cb]);
        epi.nq[cb] = epi.qv[cb] ? a.nrm_q[qs] : 0.f;
        epi.qrow[cb] = (int32_t)q;
        epi.cap[cb] = epi.qv[cb] ? a.tau[qs] : -INFINITY;
    }
    // the first database tile of the query tile's own block, and this split's share of the rest
    const int64_t f = qt * (QT / T::TR);
    const int64_t len = a.tiles - f;
    const int64_t tb = f + len * split / a.splits, te = f + len * (split + 1) / a.splits;

    epi.init();
    epi.g = g;
    epi.sv = nullptr; // no stash: the slow paths select the dot products from registers
    epi.tid = tid;
    epi.col_from = qbase + QT;
    epi.colbuf = a.colbuf;
    epi.colcnt = a.colcnt;
    epi.colcap = a.colcap;
    // the row side's bound starts at tau (prepare() re-forms it once a list changes)
    constexpr float kWiden = 1.0f / 1048576.0f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) epi.admq[cb] = fmaf(epi.cap[cb], 1.0f + kWiden, -epi.nq[cb] * (1.0f - kWiden));
    run_tiles<QM, CB, true, 1>(a.Bt, (int32_t)a.m, a.nrm_b, reinterpret_cast<const int32_t *>(a.tau), a.theta,
                               (int32_t)tb, (int32_t)te, bq, epi);

    // the row side's list of each query: this split's partial list
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        TopK<K> L;
        epi.load(cb, L);
        L.merge_xor(16);
        L.merge_xor(32);
        if (g == 0 && epi.qv[cb]) {
            Entry *dst = a.part + ((int64_t)split * a.nq + epi.qrow[cb]) * K;
#pragma unroll
            for (int t = 0; t < K; ++t) dst[t] = Entry{L.d[t], L.i[t]};
        }
    }
}

// Final lists of the symmetric pass: per row the a.splits partial lists of
// the row side and the column side's candidates (in any order, so each goes
// through the full (D2, index) comparison), kMergeLanes lanes per row as in
// knn_merge_kernel.  A row whose buffer overflowed marks its query tile in
// a.gate_w; its list is then recomputed.
template <int K> __global__ __launch_bounds__(256) void sym_merge_kernel(KnnArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ql = gid / kMergeLanes;
    const int r = (int)(gid % kMergeLanes);
    const bool row = ql < a.nq;
    TopK<K> L;
    L.clear();
    for (int s0 = 0; s0 < a.splits; s0 += kMergeLanes) {
        const int s = s0 + r;
        float od[K];
        int32_t oi[K];
        const bool have = row && s < a.splits;
        const Entry *src = a.part + ((int64_t)(have ? s : 0) * a.nq + (have ? ql : 0)) * K;
#pragma unroll
        for (int t = 0; t < K; ++t) {
            const Entry e = have ? src[t] : Entry{INFINITY, 0x7fffffff};
            od[t] = e.d2;
            oi[t] = e.idx;
        }
        L.push_sorted(od, oi);
    }
    const uint32_t cnt = row ? a.colcnt[ql] : 0u;
    const uint32_t use = cnt < (uint32_t)a.colcap ? cnt : (uint32_t)a.colcap;
    const Entry *cand = a.colbuf + (row ? ql : 0) * a.colcap;
    for (uint32_t e0 = 0; e0 < (uint32_t)a.colcap; e0 += kMergeLanes) {
        const bool h = e0 + (uint32_t)r < use;
        if (!__builtin_amdgcn_ballot_w64(h)) break;
        if (h) {
            const Entry e = cand[e0 + r];
            L.push_any(e.d2, e.idx);
        }
    }
#pragma unroll
    for (int mask = 1; mask < kMergeLanes; mask <<= 1) L.merge_xor(mask);
    if (row && r == 0) {
        write_list<K>(a, L, ql, 0);
        if (cnt > (uint32_t)a.colcap) atomicOr(&a.gate_w[ql / a.gate_rows], 1u);
    }
}

// Direct-difference D2 of the selected neighbours, for the reported kNN
// distances and the core distances: sum_f (q_f - y_f)^2 with fmaf in feature
// order, which carries no cancellation error.  One lane per (row, list entry)
// "slot", kRowLanes lanes per row (a power of two >= K): 64 slots per wave.
// Each lane sums its own slot over the positions of the point-major layout in
// order, 16 (one chunk) at a time, from LDS: the wave first stages the chunk
// of every slot's neighbour (its 64 bytes of the point-major copy Bt, read by
// four adjacent lanes, so a load instruction touches 16 cache lines instead
// of 64) and the same positions of its rows' query features (feature-major
// source), with the next two chunks' loads already in flight.  Positions run
// through the features in order; the padding positions are zero on both sides
// and add exact zeros.  The row's order is then taken across its lanes by ranks (shuffles),
// with no sort network.
template <int K> struct DirectRows {
    static constexpr int kRowLanes = K <= 16 ? 16 : 32;
    static constexpr int kRowsPerWave = 64 / kRowLanes;
    static constexpr int kRowsPerBlock = kRowsPerWave * 4; // 256 threads
};
constexpr int kDirectMaxDim = 256; // EKH_MAX_DIM rounded to 16
// floats per staged 16-feature row: 4 floats of padding make the 16-byte reads
// of 8 consecutive slots fall on distinct banks
constexpr int kSlotStride = 20;
// per wave: 64 slot rows, then up to 4 query rows
constexpr int kDirectWaveFloats = (64 + 4) * kSlotStride;
constexpr int kDirectBlockFloats = 4 * kDirectWaveFloats; // LDS of a direct-difference workgroup

// D2 of this lane's slot (row q, entry t) and its key; returns false for lanes
// past the rows.  lds: kDirectBlockFloats floats.
template <int K>
__device__ __forceinline__ bool direct_d2(const KnnArgs &a, float *lds, int64_t &q, int &t, int32_t &jo, float &d2) {
    using R = DirectRows<K>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rw = lane / R::kRowLanes; // row within the wave
    t = lane % R::kRowLanes;
    const int64_t qb = ((int64_t)blockIdx.x * 4 + wave) * R::kRowsPerWave; // first local row of the wave
    const int64_t ql = qb + rw;
    q = a.q0 + ql;
    const bool live = ql < a.nq;
    jo = (live && t < a.k_out) ? a.out_idx[q * a.k_out + t] : 0x7fffffff;
    // an entry outside [0, m) cannot come from a finished search (k <= m); it is
    // never used as an address: the slot stages zeros and ranks last
    const bool ok = live && t < a.k_out && jo >= 0 && jo < a.m;
    const int32_t jr = ok ? jo : -1;

    // loader roles: piece p of this lane is quarter (lane & 3) of slot p * 16 + lane / 4;
    // query feature (lane / rows) of the chunk for row (lane % rows)
    const int pq = lane & 3;
    const float *ysrc[4];
    bool yhas[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int32_t js = __shfl(jr, p * 16 + (lane >> 2));
        yhas[p] = js >= 0;
        ysrc[p] = a.Bt + (int64_t)(yhas[p] ? js : 0) * a.dp + 4 * pq;
    }
    const int xr = lane % R::kRowsPerWave, xf = lane / R::kRowsPerWave;
    const bool xrow = qb + xr < a.nq && xf < 16;
    const float *xsrc = a.Q + a.q0 + (xrow ? qb + xr : 0);
    const int qm = pick_qm(a.d);
    float *yw = lds + wave * kDirectWaveFloats; // [64][kSlotStride]
    float *xw = yw + 64 * kSlotStride;          // [rows][kSlotStride]

    auto load = [&](int c, f4 (&yv)[4], float &xv) {
#pragma unroll
        for (int p = 0; p < 4; ++p) yv[p] = yhas[p] ? *reinterpret_cast<const f4 *>(ysrc[p] + c * 16) : f4{0.f, 0.f, 0.f, 0.f};
        // the query feature at this position of the point-major layout (none: zero)
        const int f = pm_feature(c * 16 + xf, qm, a.d);
        xv = (xrow && f >= 0) ? xsrc[(int64_t)f * a.ldq] : 0.f;
    };
    const int nc = a.dp / 16;
    f4 ya[4], yb[4];
    float xa, xb = 0.f;
    load(0, ya, xa);
    if (nc > 1) load(1, yb, xb);
    const f4 *ymine = reinterpret_cast<const f4 *>(yw + lane * kSlotStride);
    const f4 *xmine = reinterpret_cast<const f4 *>(xw + rw * kSlotStride);
    float s = 0.f;
    for (int c = 0; c < nc; ++c) {
#pragma unroll
        for (int p = 0; p < 4; ++p) *reinterpret_cast<f4 *>(yw + (p * 16 + (lane >> 2)) * kSlotStride + 4 * pq) = ya[p];
        if (xf < 16) xw[xr * kSlotStride + xf] = xa;
        // the stores above before this wave's reads below (LDS runs one wave's
        // operations in order; this keeps the compiler from moving them)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < 4; ++p) ya[p] = yb[p];
        xa = xb;
        if (c + 2 < nc) load(c + 2, yb, xb);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f4 yv = ymine[j], xv = xmine[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = xv[e] - yv[e];
                s = fmaf(v, v, s);
            }
        }
        // this chunk's reads before the next chunk's stores
        __builtin_amdgcn_wave_barrier();
    }
    d2 = ok ? s : INFINITY;
    return live;
}

// Rank of this lane's (d2, index) among its row's lanes (lanes past k_out hold
// (inf, INT_MAX)); ties of equal keys go to the lower lane.
template <int K> __device__ __forceinline__ int direct_rank(float d2, int32_t jo, int t) {
    using R = DirectRows<K>;
    const int base = (threadIdx.x & 63) & ~(R::kRowLanes - 1);
    int rank = 0;
#pragma unroll
    for (int u = 0; u < R::kRowLanes; ++u) {
        const float du = __shfl(d2, base + u);
        const int32_t ju = __shfl(jo, base + u);
        rank += (du < d2 || (du == d2 && (ju < jo || (ju == jo && u < t)))) ? 1 : 0;
    }
    return rank;
}

// Reported kNN distances: each row's entries re-ordered by (direct D2, index)
// and reported as sqrt_rn of the direct D2.  The neighbour set itself is the
// one the GEMM-form D2 selected.
template <int K> __global__ __launch_bounds__(256) void knn_rescore_kernel(KnnArgs a) {
    __shared__ __align__(16) float lds[kDirectBlockFloats];
    int64_t q;
    int t;
    int32_t jo = 0x7fffffff;
    float d2 = INFINITY;
    const bool live = direct_d2<K>(a, lds, q, t, jo, d2);
    const int rank = direct_rank<K>(d2, jo, t); // every lane takes part in the shuffles
    if (!live || t >= a.k_out) return;
    // every lane has read its own entry before any lane of the row writes (the
    // ranks' shuffles order them), and the row's lanes lie in one wave
    a.out_idx[q * a.k_out + rank] = jo;
    if (a.out_dist) a.out_dist[q * a.k_out + rank] = sqrt_rn(d2);
}

// Core distances by direct differences: core = sqrt_rn of the min_samples-th
// smallest direct D2 among the row's K = min_samples + 1 list entries.  The list
// was selected with the GEMM-form D2; its first min_samples + 1 entries hold
// every point within the true rank-min_samples distance unless the GEMM form's
// rounding exceeds the gap between ranks min_samples and min_samples + 2, so
// this is the float32 value of the exact core distance ("HDBSCAN" page, "The
// algorithm on the device": the distance to the min_samples-th neighbour, the
// point itself counted).
template <int K> __global__ __launch_bounds__(256) void knn_core_kernel(KnnArgs a) {
    __shared__ __align__(16) float lds[kDirectBlockFloats];
    int64_t q;
    int t;
    int32_t jo = 0x7fffffff;
    float d2 = INFINITY;
    const bool live = direct_d2<K>(a, lds, q, t, jo, d2);
    const int rank = direct_rank<K>(d2, jo, t);
    if (live && t < a.k_out && rank == a.min_samples - 1) a.out_core[q] = sqrt_rn(d2);
}

template <int K> hipError_t launch_knn_tile_k(int QM, const KnnArgs &a, hipStream_t s);
template <int K> hipError_t launch_knn_rescore_k(const KnnArgs &a, hipStream_t s);
template <int K> hipError_t launch_knn_core_k(const KnnArgs &a, hipStream_t s);
template <int K> hipError_t launch_knn_merge_k(const KnnArgs &a, hipStream_t s);
template <int K> hipError_t launch_knn_sym_k(int QM, const KnnArgs &a, hipStream_t s);
template <int K> hipError_t launch_sym_merge_k(const KnnArgs &a, hipStream_t s);

} // namespace ekh
