// Per-round Boruvka kernels of libekh ("HDBSCAN" page, "The algorithm on the
// device": in a round, each component finds the lightest edge that leaves it,
// and the components joined by those edges merge; edges are ordered by
// (weight, lower index, higher index)).  All of them are O(n) memory passes; the O(|active| n) part is the
// MFMA scan in tile_kernels.hip.  Only integer atomics are used, so every
// result is independent of execution order.
#include "ekh_internal.h"

#include <hipcub/hipcub.hpp>

#include <math.h>

namespace ekh {

static inline dim3 grid_for(int64_t n, int bs) { return dim3((unsigned)((n + bs - 1) / bs)); }
typedef float f4v __attribute__((ext_vector_type(4)));
constexpr int kBs = 256;
// Per-point passes whose atomics go to few addresses late in the run (a
// component's minimum, a global counter) combine them per workgroup in LDS
// first: 1,024 points per workgroup, one global atomic per workgroup and label.
constexpr int kBigBs = 1024;
constexpr int kHashBits = 11;
constexpr int kHashSlots = 1 << kHashBits; // > kBigBs: the table of one workgroup never fills

__global__ void bv_init_kernel(BvState st) {
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a >= st.n) return;
    st.comp[a] = (int32_t)a;
    st.cc[a] = ((uint64_t)(uint32_t)a << 32) | __float_as_uint(st.core[a]);
    st.parent[a] = (int32_t)a;
    st.cmin1[a] = kNoEdge;
    st.cmin2[a] = 0xffffffffu;
    st.compW[a] = kInfBits;
    st.csize[a] = 0;
    if (a == 0) *st.ctr = BvCounters{};
}

hipError_t bv_init(const BvState &st, hipStream_t s) {
    hipLaunchKernelGGL(bv_init_kernel, grid_for(st.n, kBs), dim3(kBs), 0, s, st);
    return hipGetLastError();
}

// The per-round counters; ctr->giant (set at the end of the previous round by
// bv_giant) is kept.
__global__ void bv_reset_counters_kernel(BvCounters *c) {
    if (threadIdx.x == 0) {
        c->n_active = 0;
        c->n_resolved = 0;
        c->n_skipped = 0;
        c->n_roots = 0;
        c->n_missing = 0;
        c->n_active_g = 0;
        c->n_comp_g = 0;
    }
}

hipError_t bv_reset_counters(const BvState &st, hipStream_t s) {
    hipLaunchKernelGGL(bv_reset_counters_kernel, dim3(1), dim3(64), 0, s, st.ctr);
    return hipGetLastError();
}

// Adds the number of set predicates of the wave to *ctr with one atomic.
__device__ __forceinline__ void wave_count(bool pred, uint32_t *ctr) {
    const uint64_t m = __ballot(pred);
    if ((threadIdx.x & 63) == (unsigned)__ffsll((long long)__ballot(1)) - 1 && m)
        atomicAdd(ctr, (uint32_t)__popcll(m));
}

// Per-workgroup minima (or sums, ADD) by label in LDS: open addressing with
// linear probing (label -1 = free slot).  A workgroup inserts at most kBigBs
// labels into kHashSlots > kBigBs slots, so a free slot always exists; the
// bounded probe loop falls back to the global atomic all the same.
template <class T, bool ADD = false> struct LdsMinTable {
    __device__ __forceinline__ static void op(T *p, T v) {
        if (ADD)
            atomicAdd(p, v);
        else
            atomicMin(p, v);
    }
    int32_t key[kHashSlots];
    T val[kHashSlots];

    __device__ __forceinline__ void clear() {
        for (int i = threadIdx.x; i < kHashSlots; i += blockDim.x) {
            key[i] = -1;
            val[i] = ADD ? T(0) : ~T(0);
        }
    }
    __device__ __forceinline__ void insert(int32_t c, T v, T *gbase) {
        uint32_t h = ((uint32_t)c * 2654435761u) >> (32 - kHashBits);
        for (int p = 0; p < kHashSlots; ++p) {
            const int32_t k = atomicCAS(&key[h], -1, c);
            if (k == -1 || k == c) {
                op(&val[h], v);
                return;
            }
            h = (h + 1) & (kHashSlots - 1);
        }
        op(&gbase[c], v);
    }
    // the lanes that share the wave's first label combine (wave minimum or sum)
    // and insert once; the others insert their own
    __device__ __forceinline__ void insert_grouped(int32_t c, T v, bool active, T *gbase) {
        const uint64_t act = __ballot(active);
        if (!act) return;
        const int lane = threadIdx.x & 63;
        const int leader = __ffsll((long long)act) - 1;
        const int32_t c0 = __shfl(c, leader);
        const bool same = active && c == c0;
        T m = same ? v : (ADD ? T(0) : ~T(0));
        for (int o = 32; o > 0; o >>= 1) {
            const T y = __shfl_xor(m, o);
            m = ADD ? m + y : (y < m ? y : m);
        }
        if (lane == leader) insert(c0, m, gbase);
        if (active && !same) insert(c, v, gbase);
    }
    // after a barrier: one global atomic per label the workgroup saw
    __device__ __forceinline__ void flush(T *gbase) {
        for (int i = threadIdx.x; i < kHashSlots; i += blockDim.x)
            if (key[i] >= 0) op(&gbase[key[i]], val[i]);
    }
};

// Adds the wave's set predicates to the workgroup's LDS counter (zeroed before a barrier).
__device__ __forceinline__ void lds_count(bool pred, uint32_t *cnt) {
    const uint64_t m = __ballot(pred);
    if ((threadIdx.x & 63) == 0 && m) atomicAdd(cnt, (uint32_t)__popcll(m));
}

// Neighbour-edge candidates ("Exact shortcuts", first item).  For point a with
// list entries b (self included, ascending (D2, index)), last entry at distance
// D_last:
//  - every entry in another component is a real edge W = max(core_a, core_b, D);
//    the smallest (W, b) is a's best list edge and feeds the component bound;
//  - the list holds every point closer than D_last (it is the K nearest under
//    (D2, index), with the same D2 the scan computes), so every edge of a to a
//    point outside the list weighs at least max(core_a, D_last).  A best list
//    edge lighter than D_last is therefore a's cheapest edge, and a is resolved
//    without a scan.  This contains the page's case (W == core_a with the last
//    entry, the extra (min_samples + 1)-th neighbour, strictly farther than
//    core_a) and extends it to any best list edge below D_last;
//  - a point that is not resolved has no edge lighter than
//    lb = max(core_a, D_last) (its list edges are >= the best one >= D_last):
//    lb goes to the activity pass, which compares it with the component bound.
// With use_nb = 0 neither list argument is used (lb = core_a, which bounds
// every edge of a by the definition of W).
__global__ __launch_bounds__(kBigBs) void bv_candidates_kernel(BvState st, int use_nb, int use_bound) {
    __shared__ LdsMinTable<uint32_t> tab;
    __shared__ uint32_t n_res;
    tab.clear();
    if (threadIdx.x == 0) n_res = 0;
    __syncthreads();
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool res = false, bnd = false;
    uint32_t wb = 0;
    int32_t cb = 0;
    if (a < st.n) {
        const int32_t ca = st.comp[a];
        const float corea = st.core[a];
        uint64_t nb = kNoEdge;
        float last_d2 = 0.f;
        for (int t = 0; t < st.K; ++t) {
            const int32_t b = st.nbr_idx[a * st.K + t];
            const float d2 = st.nbr_d2[a * st.K + t];
            last_d2 = d2;
            if (b < 0 || b >= st.n) continue; // malformed caller list: entry ignored
            const uint64_t x = st.cc[b];        // comp << 32 | core bits of b
            if ((int32_t)(x >> 32) != ca) {
                const float D = sqrt_rn(d2 > 0.f ? d2 : 0.f);
                const float W = fmaxf(fmaxf(corea, __uint_as_float((uint32_t)x)), D);
                const uint64_t key = ((uint64_t)__float_as_uint(W) << 32) | (uint32_t)b;
                nb = key < nb ? key : nb;
            }
        }
        const float dlast = sqrt_rn(last_d2 > 0.f ? last_d2 : 0.f);
        res = use_nb && nb != kNoEdge && __uint_as_float((uint32_t)(nb >> 32)) < dlast;
        st.best[a] = nb;
        st.resolved[a] = res ? 1 : 0;
        st.lbound[a] = use_nb ? fmaxf(corea, dlast) : corea;
        bnd = use_bound && nb != kNoEdge;
        wb = (uint32_t)(nb >> 32);
        cb = ca;
    }
    tab.insert_grouped(cb, wb, bnd, st.compW);
    lds_count(res, &n_res);
    __syncthreads();
    tab.flush(st.compW);
    if (threadIdx.x == 0 && n_res) atomicAdd(&st.ctr->n_resolved, n_res);
}

hipError_t bv_candidates(const BvState &st, int use_nb, int use_bound, hipStream_t s) {
    hipLaunchKernelGGL(bv_candidates_kernel, grid_for(st.n, kBigBs), dim3(kBigBs), 0, s, st, use_nb, use_bound);
    return hipGetLastError();
}

// Active points ("Exact shortcuts", second item): not resolved, and not skipped
// by the component bound (a point whose lower bound lb (core_a, or
// max(core_a, D_last) from its list, see bv_candidates_kernel) exceeds the
// lightest known edge out of its component cannot supply a lighter one; on
// equality it still could, through a lower index, so it stays active).
// Compacted into st.act with one atomic per wave.
// Appends the lanes with `take` to list[] at positions claimed with one
// atomic per wave on *count.
__device__ __forceinline__ void wave_append(bool take, int32_t value, uint32_t *count, int32_t *list) {
    const uint64_t m = __ballot(take);
    const int lane = threadIdx.x & 63;
    uint32_t base = 0;
    if (lane == 0 && m) base = atomicAdd(count, (uint32_t)__popcll(m));
    base = __shfl(base, 0);
    if (take) list[base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull))] = value;
}

// With split_giant, the active points of the largest component (when it holds
// at least half of the points) go to act_g instead: they need to be scanned
// only against the points outside it.
__global__ __launch_bounds__(kBigBs) void bv_select_active_kernel(BvState st, int use_bound, int split_giant) {
    __shared__ uint32_t n_skip;
    if (threadIdx.x == 0) n_skip = 0;
    __syncthreads();
    const uint64_t gk = split_giant ? st.ctr->giant : 0;
    const bool use_g = split_giant && (gk >> 32) * 2 >= (uint64_t)st.n;
    const int32_t g = (int32_t)(uint32_t)gk;
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool act = false, skip = false, in_g = false;
    if (a < st.n && !st.resolved[a]) {
        const int32_t c = st.comp[a];
        skip = use_bound && st.lbound[a] > __uint_as_float(st.compW[c]);
        act = !skip;
        in_g = use_g && c == g;
    }
    wave_append(act && !in_g, (int32_t)a, &st.ctr->n_active, st.act);
    wave_append(act && in_g, (int32_t)a, &st.ctr->n_active_g, st.act_g);
    lds_count(skip, &n_skip);
    __syncthreads();
    if (threadIdx.x == 0 && n_skip) atomicAdd(&st.ctr->n_skipped, n_skip);
}

hipError_t bv_select_active(const BvState &st, int use_bound, int split_giant, hipStream_t s) {
    hipLaunchKernelGGL(bv_select_active_kernel, grid_for(st.n, kBigBs), dim3(kBigBs), 0, s, st, use_bound,
                       split_giant);
    return hipGetLastError();
}

// Size of every component (LDS-combined counts per label), then the largest
// as size << 32 | label (ties to the larger label) in ctr->giant.  Run after a
// round's relabel (csize is zero then), for the next round.
__global__ __launch_bounds__(kBigBs) void bv_comp_sizes_kernel(BvState st) {
    __shared__ LdsMinTable<uint32_t, true> tab;
    if (blockIdx.x == 0 && threadIdx.x == 0) st.ctr->giant = 0; // bv_giant_kernel, launched next, accumulates it
    tab.clear();
    __syncthreads();
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool in = a < st.n;
    tab.insert_grouped(in ? st.comp[a] : 0, 1u, in, st.csize);
    __syncthreads();
    tab.flush(st.csize);
}

__global__ __launch_bounds__(kBigBs) void bv_giant_kernel(BvState st) {
    __shared__ unsigned long long bmax;
    if (threadIdx.x == 0) bmax = 0;
    __syncthreads();
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned long long k = 0;
    if (a < st.n && st.comp[a] == (int32_t)a) k = ((unsigned long long)st.csize[a] << 32) | (uint32_t)a;
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long y = __shfl_xor(k, o);
        k = y > k ? y : k;
    }
    if ((threadIdx.x & 63) == 0 && k) atomicMax(&bmax, k);
    __syncthreads();
    if (threadIdx.x == 0 && bmax) atomicMax((unsigned long long *)&st.ctr->giant, bmax);
}

hipError_t bv_giant(const BvState &st, hipStream_t s) {
    hipLaunchKernelGGL(bv_comp_sizes_kernel, grid_for(st.n, kBigBs), dim3(kBigBs), 0, s, st);
    hipLaunchKernelGGL(bv_giant_kernel, grid_for(st.n, kBigBs), dim3(kBigBs), 0, s, st);
    return hipGetLastError();
}

// The points outside component `giant`, listed in orig (ctr->n_comp_g of
// them); one atomic per workgroup, waves placed by an LDS prefix.
// Nothing to do when the round lists no active point of that component.
__global__ __launch_bounds__(kBigBs) void bv_complement_kernel(BvState st, int32_t giant, int32_t *orig) {
    __shared__ uint32_t wcount[kBigBs / 64];
    __shared__ uint32_t base;
    if (__hip_atomic_load(&st.ctr->n_active_g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool out = a < st.n && st.comp[a] != giant;
    const uint64_t m = __ballot(out);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) wcount[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kBigBs / 64; ++w) {
            const uint32_t c = wcount[w];
            wcount[w] = t;
            t += c;
        }
        base = t ? atomicAdd(&st.ctr->n_comp_g, t) : 0;
    }
    __syncthreads();
    if (out) orig[base + wcount[wave] + (uint32_t)__popcll(m & ((1ull << lane) - 1ull))] = (int32_t)a;
}

hipError_t bv_complement(const BvState &st, int32_t giant, int32_t *orig, hipStream_t s) {
    hipLaunchKernelGGL(bv_complement_kernel, grid_for(st.n, kBigBs), dim3(kBigBs), 0, s, st, giant, orig);
    return hipGetLastError();
}

// Feature-major copy [d, ns] of the listed points with their norms, core
// distances and labels (writes coalesced along the list).  Only the first
// *count (<= ns) list entries are read; with *gate == 0 nothing is done.
// One thread per 16-byte piece of a gathered row (dp / 4 pieces per row, so a
// wave copies whole rows contiguously); the row's first thread also copies its
// norm, core distance and label.
__global__ __launch_bounds__(kBs) void bv_gather_points_kernel(const float *P, int dp, const int32_t *orig,
                                                                int64_t ns, const float *nrm, const float *core,
                                                                const int32_t *comp, float *xs, float *nrm_s,
                                                                float *core_s, int32_t *comp_s, const uint32_t *count,
                                                                const uint32_t *gate) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gate && __hip_atomic_load(gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) return;
    const int64_t listed = count ? (int64_t)__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : ns;
    const int ppr = dp / 4;
    const int64_t i = t / ppr;
    const int piece = (int)(t - i * ppr);
    if (i >= ns) return;
    f4v *dst = reinterpret_cast<f4v *>(xs + i * dp) + piece;
    if (i >= listed) {
        // fewer points listed than the host sized the copy for (it reports the
        // mismatch after the round): such rows carry the padding label and
        // never form an edge
        *dst = f4v{0.f, 0.f, 0.f, 0.f};
        if (piece == 0) {
            nrm_s[i] = INFINITY;
            core_s[i] = INFINITY;
            comp_s[i] = -1;
        }
        return;
    }
    const int32_t p = orig[i];
    *dst = reinterpret_cast<const f4v *>(P + (int64_t)p * dp)[piece];
    if (piece == 0) {
        nrm_s[i] = nrm[p];
        core_s[i] = core[p];
        comp_s[i] = comp[p];
    }
}

hipError_t bv_gather_points(const float *P, int dp, const int32_t *orig, int64_t ns, const float *nrm,
                            const float *core, const int32_t *comp, float *xs, float *nrm_s, float *core_s,
                            int32_t *comp_s, const uint32_t *count, const uint32_t *gate, hipStream_t s) {
    if (ns <= 0) return hipSuccess;
    if (dp <= 0 || dp % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bv_gather_points_kernel, grid_for(ns * (dp / 4), kBs), dim3(kBs), 0, s, P, dp, orig, ns, nrm,
                       core, comp, xs, nrm_s, core_s, comp_s, count, gate);
    return hipGetLastError();
}

// Component minimum of (W, lo, hi) over the members' best edges: the 70-bit key
// is reduced in two integer passes, (W bits << 32 | lo) first, then hi among
// the edges that reach that minimum.
__global__ __launch_bounds__(kBigBs) void bv_cmin1_kernel(BvState st) {
    __shared__ LdsMinTable<unsigned long long> tab;
    tab.clear();
    __syncthreads();
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool has = false;
    unsigned long long key = 0;
    int32_t c = 0;
    if (a < st.n) {
        const uint64_t k = st.best[a];
        if (k != kNoEdge) {
            const uint32_t b = (uint32_t)k;
            const uint32_t lo = (uint32_t)a < b ? (uint32_t)a : b;
            key = (unsigned long long)((k & 0xffffffff00000000ull) | lo);
            c = st.comp[a];
            has = true;
        }
    }
    tab.insert_grouped(c, key, has, (unsigned long long *)st.cmin1);
    __syncthreads();
    tab.flush((unsigned long long *)st.cmin1);
}

__global__ void bv_cmin2_kernel(BvState st) {
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a >= st.n) return;
    const uint64_t k = st.best[a];
    if (k == kNoEdge) return;
    const uint32_t b = (uint32_t)k;
    const uint32_t lo = (uint32_t)a < b ? (uint32_t)a : b, hi = (uint32_t)a < b ? b : (uint32_t)a;
    const int32_t c = st.comp[a];
    if (((k & 0xffffffff00000000ull) | lo) == st.cmin1[c]) atomicMin(&st.cmin2[c], hi);
}

hipError_t bv_component_min(const BvState &st, hipStream_t s) {
    hipLaunchKernelGGL(bv_cmin1_kernel, grid_for(st.n, kBigBs), dim3(kBigBs), 0, s, st);
    hipLaunchKernelGGL(bv_cmin2_kernel, grid_for(st.n, kBs), dim3(kBs), 0, s, st);
    return hipGetLastError();
}

// Each component c (label = its root point, comp[c] == c) takes its cheapest
// edge to component c2.  If c2 chose the same edge (a mutual pair) the edge is
// kept once, by the smaller label, which stays a root; every other component
// hooks onto c2.  With a strict edge order these are the only cycles.
__global__ void bv_select_edges_kernel(BvState st) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= st.n || st.comp[c] != (int32_t)c) return;
    const uint64_t k1 = st.cmin1[c];
    if (k1 == kNoEdge) {
        atomicAdd(&st.ctr->n_missing, 1u);
        st.parent[c] = (int32_t)c;
        return;
    }
    const int32_t lo = (int32_t)(uint32_t)k1;
    const int32_t hi = (int32_t)st.cmin2[c];
    const int32_t other = st.comp[lo] == (int32_t)c ? hi : lo;
    const int32_t c2 = st.comp[other];
    const bool mutual = st.cmin1[c2] == k1 && st.cmin2[c2] == (uint32_t)hi;
    if (mutual && (int32_t)c > c2) {
        st.parent[c] = c2; // the partner records the edge
        return;
    }
    st.parent[c] = mutual ? (int32_t)c : c2;
    const uint32_t pos = atomicAdd(&st.ctr->n_edges, 1u);
    if ((int64_t)pos >= st.n) return; // cannot happen for a strict edge order; the host reports the count
    st.e_lo[pos] = lo;
    st.e_hi[pos] = hi;
    st.e_w[pos] = __uint_as_float((uint32_t)(k1 >> 32));
}

hipError_t bv_select_edges(const BvState &st, hipStream_t s) {
    hipLaunchKernelGGL(bv_select_edges_kernel, grid_for(st.n, kBs), dim3(kBs), 0, s, st);
    return hipGetLastError();
}

// One pointer-jumping step over the roots of the previous round: parent[c] =
// parent[parent[c]].  The host runs a fixed ceil(log2(components)) + 1 steps,
// enough for any hook tree.  In-place updates only move pointers further up.
__global__ void bv_jump_kernel(BvState st) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= st.n || st.comp[c] != (int32_t)c) return;
    st.parent[c] = st.parent[st.parent[c]];
}

hipError_t bv_jump(const BvState &st, hipStream_t s) {
    hipLaunchKernelGGL(bv_jump_kernel, grid_for(st.n, kBs), dim3(kBs), 0, s, st);
    return hipGetLastError();
}

// New label of every point = the root its old component hooked to; counts the
// surviving roots and clears the per-component arrays for the next round.
__global__ void bv_relabel_kernel(BvState st) {
    const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool root = false;
    if (a < st.n) {
        const int32_t c = st.comp[a];
        const int32_t r = st.parent[c];
        root = (c == (int32_t)a) && (r == (int32_t)a);
        st.comp[a] = r;
        st.cc[a] = ((uint64_t)(uint32_t)r << 32) | __float_as_uint(st.core[a]);
        st.cmin1[a] = kNoEdge;
        st.cmin2[a] = 0xffffffffu;
        st.compW[a] = kInfBits;
        st.csize[a] = 0;
    }
    wave_count(root, &st.ctr->n_roots);
}

hipError_t bv_relabel(const BvState &st, hipStream_t s) {
    hipLaunchKernelGGL(bv_relabel_kernel, grid_for(st.n, kBs), dim3(kBs), 0, s, st);
    return hipGetLastError();
}

// Reported weight of every tree edge: max(core_lo, core_hi, D) with D by direct
// differences, sqrt_rn(sum_f (x_lo,f - x_hi,f)^2) with fmaf in feature order,
// from a point-major copy P [n, dp] (zero padding features add exact zeros).
// The tree was chosen with the GEMM-form D (the value the candidate pass and
// the scan share bit for bit); the two differ by its rounding only, which the
// direct form does not carry.  Symmetric in (lo, hi) bit for bit.
__global__ void bv_edge_weights_kernel(const float *__restrict__ P, int dp, const float *__restrict__ core,
                                       const int32_t *__restrict__ lo, const int32_t *__restrict__ hi, int64_t ne,
                                       int64_t n, float *__restrict__ w) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ne) return;
    const int32_t a = lo[i], b = hi[i];
    if (a < 0 || a >= n || b < 0 || b >= n) { // cannot come from a finished tree
        w[i] = INFINITY;
        return;
    }
    const f4 *pa = reinterpret_cast<const f4 *>(P + (int64_t)a * dp);
    const f4 *pb = reinterpret_cast<const f4 *>(P + (int64_t)b * dp);
    float s = 0.f;
#pragma unroll 4
    for (int f = 0; f < dp / 4; ++f) {
        const f4 x = pa[f], y = pb[f];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = x[e] - y[e];
            s = fmaf(v, v, s);
        }
    }
    w[i] = fmaxf(fmaxf(core[a], core[b]), sqrt_rn(s));
}

hipError_t bv_edge_weights(const float *P, int dp, const float *core, const int32_t *lo, const int32_t *hi, int64_t ne,
                           int64_t n, float *w, hipStream_t s) {
    if (ne <= 0) return hipSuccess;
    hipLaunchKernelGGL(bv_edge_weights_kernel, grid_for(ne, kBs), dim3(kBs), 0, s, P, dp, core, lo, hi, ne, n, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------- edge sort
// Order (W, lo, hi): a stable radix sort by hi, then a stable one by
// (W bits << 32 | lo) -- W >= 0, so its bits order like the values.
__global__ void es_prep1(const int32_t *hi, int64_t ne, uint32_t *key, uint32_t *val) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ne) return;
    key[i] = (uint32_t)hi[i];
    val[i] = (uint32_t)i;
}
__global__ void es_prep2(const int32_t *lo, const float *w, const uint32_t *perm, int64_t ne, uint64_t *key) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ne) return;
    const uint32_t e = perm[i];
    key[i] = ((uint64_t)__float_as_uint(w[e]) << 32) | (uint32_t)lo[e];
}
__global__ void es_gather(const int32_t *lo, const int32_t *hi, const float *w, const uint32_t *perm, int64_t ne,
                          int32_t *olo, int32_t *ohi, float *ow) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= ne) return;
    const uint32_t e = perm[i];
    olo[i] = lo[e];
    ohi[i] = hi[e];
    ow[i] = w[e];
}

size_t edge_sort_temp_bytes(int64_t ne) {
    size_t b1 = 0, b2 = 0;
    if (ne <= 0) return 16;
    hipcub::DeviceRadixSort::SortPairs(nullptr, b1, (const uint32_t *)nullptr, (uint32_t *)nullptr,
                                       (const uint32_t *)nullptr, (uint32_t *)nullptr, (int)ne);
    hipcub::DeviceRadixSort::SortPairs(nullptr, b2, (const uint64_t *)nullptr, (uint64_t *)nullptr,
                                       (const uint32_t *)nullptr, (uint32_t *)nullptr, (int)ne);
    return (b1 > b2 ? b1 : b2) + 16;
}

hipError_t edge_sort(const int32_t *lo, const int32_t *hi, const float *w, int64_t ne, void *tmp, size_t tmp_bytes,
                     uint32_t *ka, uint32_t *kb, uint32_t *va, uint32_t *vb, uint64_t *k64a, uint64_t *k64b,
                     int32_t *out_lo, int32_t *out_hi, float *out_w, hipStream_t s) {
    if (ne <= 0) return hipSuccess;
    const dim3 g = grid_for(ne, kBs);
    hipLaunchKernelGGL(es_prep1, g, dim3(kBs), 0, s, hi, ne, ka, va);
    size_t tb = tmp_bytes;
    hipError_t e = hipcub::DeviceRadixSort::SortPairs(tmp, tb, ka, kb, va, vb, (int)ne, 0, 32, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(es_prep2, g, dim3(kBs), 0, s, lo, w, vb, ne, k64a);
    tb = tmp_bytes;
    e = hipcub::DeviceRadixSort::SortPairs(tmp, tb, k64a, k64b, vb, va, (int)ne, 0, 64, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(es_gather, g, dim3(kBs), 0, s, lo, hi, w, va, ne, out_lo, out_hi, out_w);
    return hipGetLastError();
}

} // namespace ekh
