// Bipartite kNN-graph assignment of libekh (ekh_bipartite_assign).
//
// Kilosort4 clustering page, section "Assignment in parallel: why the graph is
// bipartite".  The graph has the spikes on one side and a copy of the subset on
// the other, with one edge per kNN link.  Once the subset's labels are held
// fixed, no spike's choice affects another's, so every spike is relabelled in
// one parallel step (left step); the subset side is then relabelled the same
// way (right step), and the two steps alternate.  The right
// step counts labels with integer atomics into counts[r, label]; each thread
// takes the label maximising n - gamma k K_c / 2m; one counter of moved spikes
// is read back per round.  The conventions the page leaves open are listed in
// include/ekh.h.  Integer atomics only, so every result is independent of the
// order in which the atomics land.
#include "ekh.h"
#include "host_error.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

namespace {

constexpr int kBs = 256;
constexpr int kMaxK = 32;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return ekh::report_error(code, buf);
}

#define BP_HIP(call)                                                                                                   \
    do {                                                                                                               \
        hipError_t e_ = (call);                                                                                        \
        if (e_ != hipSuccess) return fail(EKH_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));                    \
    } while (0)

dim3 grid_for(int64_t count) { return dim3((unsigned)((count + kBs - 1) / kBs)); }

// score n - gamma k K / (2 m), float64, in this order (no contraction: no
// multiply feeds an add)
__device__ __forceinline__ double score(uint32_t n_c, uint32_t k_v, uint32_t K_c, double two_m, double gamma) {
    return (double)n_c - gamma * (double)k_v * (double)K_c / two_m;
}

__device__ __forceinline__ void count_wave(bool flag, uint32_t *ctr) {
    const uint64_t b = __ballot(flag);
    if ((threadIdx.x & 63) == (__ffsll((long long)__ballot(1)) - 1) && b) atomicAdd(ctr, (uint32_t)__popcll(b));
}

__global__ void bp_fill(uint32_t *p, int64_t count, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = v;
}

// bad[0]: neighbour indices outside [0, m); bad[1]: starting labels outside [0, C)
__global__ void bp_check(const int32_t *nbr, int64_t edges, int64_t m, const int32_t *init, int64_t C, uint32_t *bad) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    count_wave(i < edges && (nbr[i] < 0 || nbr[i] >= m), &bad[0]);
    count_wave(i < m && (init[i] < 0 || init[i] >= C), &bad[1]);
}

__global__ void bp_degree(const int32_t *nbr, int64_t edges, uint32_t *deg) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < edges) atomicAdd(&deg[nbr[e]], 1u);
}

__global__ void bp_copy_labels(const int32_t *src, int64_t count, int32_t *dst) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) dst[i] = src[i];
}

// Histograms with few bins (the label totals, the cluster edge counts) put
// many atomics on few addresses.  With at most kLdsBins bins each block first
// counts into LDS and then adds its non-zero bins once; the block count is set
// so that a block sees several items per bin.  Integer sums: the result does
// not depend on the order.
constexpr int kLdsBins = 8192;   // 32 KB of LDS
constexpr int kHistMaxBlocks = 256;

// K_right[c] = total degree of the right nodes labelled c
struct RightTotals {
    const int32_t *right;
    const uint32_t *deg;
    __device__ uint32_t bin(int64_t r) const { return (uint32_t)right[r]; }
    __device__ uint32_t weight(int64_t r) const { return deg[r]; }
};

// cnt_left[c] = spikes labelled c (their total degree is k cnt_left[c])
struct LeftCounts {
    const int32_t *left;
    __device__ uint32_t bin(int64_t i) const { return (uint32_t)left[i]; }
    __device__ uint32_t weight(int64_t) const { return 1u; }
};

// counts[left(i) * C + right(r)] += 1 for every edge (i, r)
struct EdgeBins {
    const int32_t *nbr, *left, *right;
    int k;
    int64_t C;
    __device__ uint32_t bin(int64_t e) const { return (uint32_t)((int64_t)left[e / k] * C + right[nbr[e]]); }
    __device__ uint32_t weight(int64_t) const { return 1u; }
};

template <class F>
__global__ __launch_bounds__(kBs) void bp_hist_lds(F f, int64_t items, int bins, uint32_t *out) {
    __shared__ uint32_t h[kLdsBins];
    for (int b = threadIdx.x; b < bins; b += kBs) h[b] = 0;
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * kBs + threadIdx.x; i < items; i += (int64_t)gridDim.x * kBs) {
        const uint32_t w = f.weight(i);
        if (w) atomicAdd(&h[f.bin(i)], w);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < bins; b += kBs)
        if (h[b]) atomicAdd(&out[b], h[b]);
}

template <class F>
__global__ __launch_bounds__(kBs) void bp_hist_global(F f, int64_t items, uint32_t *out) {
    const int64_t i = (int64_t)blockIdx.x * kBs + threadIdx.x;
    if (i < items) {
        const uint32_t w = f.weight(i);
        if (w) atomicAdd(&out[f.bin(i)], w);
    }
}

// out[f.bin(i)] += f.weight(i) for every item (out already cleared)
template <class F>
void histogram(F f, int64_t items, int64_t bins, uint32_t *out, hipStream_t s) {
    if (bins <= kLdsBins) {
        int64_t blocks = items / (8 * bins); // about eight items per bin and block
        blocks = blocks < 1 ? 1 : blocks > kHistMaxBlocks ? kHistMaxBlocks : blocks;
        const int64_t most = (items + kBs - 1) / kBs;
        blocks = blocks > most ? (most < 1 ? 1 : most) : blocks;
        hipLaunchKernelGGL(bp_hist_lds<F>, dim3((unsigned)blocks), dim3(kBs), 0, s, f, items, (int)bins, out);
    } else {
        hipLaunchKernelGGL(bp_hist_global<F>, grid_for(items), dim3(kBs), 0, s, f, items, out);
    }
}

// Left step: one thread per spike; its k neighbours' labels are counted in
// registers.  Candidates are the labels present; ties keep the current label
// if it is among the best, else take the smallest.
__global__ void bp_left_step(const int32_t *nbr, int64_t n, int k, const int32_t *right, const uint32_t *K_right,
                             double two_m, double gamma, int32_t *left, uint32_t *moved) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool mv = false;
    if (i < n) {
        int32_t lab[kMaxK];
        for (int t = 0; t < k; ++t) lab[t] = right[nbr[i * k + t]];
        const int32_t cur = left[i];
        double best_s = -INFINITY, cur_s = -INFINITY;
        int32_t best_c = 0x7fffffff;
        bool cur_present = false;
        for (int t = 0; t < k; ++t) {
            const int32_t c = lab[t];
            bool seen = false;
            for (int u = 0; u < t; ++u) seen |= lab[u] == c;
            if (seen) continue;
            uint32_t n_c = 0;
            for (int u = t; u < k; ++u) n_c += lab[u] == c;
            const double s = score(n_c, (uint32_t)k, K_right[c], two_m, gamma);
            if (s > best_s || (s == best_s && c < best_c)) {
                best_s = s;
                best_c = c;
            }
            if (c == cur) {
                cur_present = true;
                cur_s = s;
            }
        }
        const int32_t nl = (cur_present && cur_s == best_s) ? cur : best_c;
        mv = nl != cur;
        left[i] = nl;
    }
    count_wave(mv, moved);
}

// Right step, first part: counts[r, label(i)] += 1 for every edge (i, r)
__global__ void bp_count(const int32_t *nbr, int64_t n, int k, const int32_t *left, int64_t C, uint32_t *counts) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < n * (int64_t)k) atomicAdd(&counts[(int64_t)nbr[e] * C + left[e / k]], 1u);
}

// Right step, second part: one thread per right node over its row of counts
__global__ void bp_right_step(const uint32_t *counts, int64_t m, int64_t C, const uint32_t *deg,
                              const uint32_t *cnt_left, int k, double two_m, double gamma, int32_t *right) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= m || deg[r] == 0) return;
    const uint32_t *row = counts + r * C;
    const int32_t cur = right[r];
    double best_s = -INFINITY, cur_s = -INFINITY;
    int32_t best_c = 0x7fffffff;
    bool cur_present = false;
    for (int64_t c = 0; c < C; ++c) {
        const uint32_t n_c = row[c];
        if (!n_c) continue;
        const double s = score(n_c, deg[r], (uint32_t)k * cnt_left[c], two_m, gamma);
        if (s > best_s) { // ascending c: the first best is the smallest
            best_s = s;
            best_c = (int32_t)c;
        }
        if (c == cur) {
            cur_present = true;
            cur_s = s;
        }
    }
    right[r] = (cur_present && cur_s == best_s) ? cur : best_c;
}

// bad[0]: neighbour indices outside [0, m); bad[1]: left labels outside [0, C);
// bad[2]: right labels outside [0, C)
__global__ void bp_check_labels(const int32_t *nbr, int64_t edges, int64_t m, const int32_t *left, int64_t n,
                                const int32_t *right, int64_t C, uint32_t *bad) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    count_wave(i < edges && (nbr[i] < 0 || nbr[i] >= m), &bad[0]);
    count_wave(i < n && (left[i] < 0 || left[i] >= C), &bad[1]);
    count_wave(i < m && (right[i] < 0 || right[i] >= C), &bad[2]);
}

struct Ws {
    uint32_t *deg, *K_right, *cnt_left, *counts, *ctr; // ctr: [0] moved, [1..2] bad
    size_t bytes;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

Ws carve(void *base, int64_t m, int64_t C) {
    Ws w{};
    char *p = (char *)base;
    size_t off = 0;
    auto take = [&](size_t count) {
        uint32_t *q = p ? (uint32_t *)(p + off) : nullptr;
        off += align256(count * 4);
        return q;
    };
    w.deg = take(m);
    w.K_right = take(C);
    w.cnt_left = take(C);
    w.counts = take((size_t)m * C);
    w.ctr = take(4);
    w.bytes = off;
    return w;
}

} // namespace

extern "C" size_t ekh_bipartite_workspace_bytes(int64_t m, int32_t n_clusters) {
    if (m < 1 || n_clusters < 1) return 0;
    return carve(nullptr, m, n_clusters).bytes;
}

extern "C" int ekh_bipartite_assign(const int32_t *nbr, int64_t n, int32_t k, int64_t m, int32_t n_clusters,
                                    const int32_t *init_right, double gamma, int32_t max_rounds, int32_t *out_left,
                                    int32_t *out_right, int32_t *out_rounds, void *ws, size_t ws_bytes,
                                    void *stream) {
    if (!nbr || !init_right || !out_left || !out_right) return fail(EKH_EINVAL, "NULL array");
    if (n < 1 || m < 1) return fail(EKH_EINVAL, "n = %lld and m = %lld must be >= 1", (long long)n, (long long)m);
    if (k < 1 || k > kMaxK) return fail(EKH_EINVAL, "k = %d out of range [1, %d]", k, kMaxK);
    if (n_clusters < 1) return fail(EKH_EINVAL, "n_clusters = %d must be >= 1", n_clusters);
    if (n * (int64_t)k >= (int64_t(1) << 31)) return fail(EKH_EINVAL, "n k = %lld edges >= 2^31", (long long)(n * k));
    if (m * (int64_t)n_clusters >= (int64_t(1) << 31))
        return fail(EKH_EINVAL, "m n_clusters = %lld >= 2^31", (long long)(m * n_clusters));
    if (!(gamma >= 0.0) || std::isinf(gamma)) return fail(EKH_EINVAL, "gamma must be finite and >= 0");
    if (max_rounds < 1) return fail(EKH_EINVAL, "max_rounds must be >= 1");
    if (!ws) return fail(EKH_EINVAL, "workspace is NULL");
    const Ws w = carve(ws, m, n_clusters);
    if (ws_bytes < w.bytes) return fail(EKH_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.bytes);
    hipStream_t s = (hipStream_t)stream;
    const int64_t edges = n * (int64_t)k, C = n_clusters;
    const double two_m = 2.0 * (double)edges;
    uint32_t host[3];

    hipLaunchKernelGGL(bp_fill, grid_for(4), dim3(kBs), 0, s, w.ctr, (int64_t)4, 0u);
    hipLaunchKernelGGL(bp_check, grid_for(edges > m ? edges : m), dim3(kBs), 0, s, nbr, edges, m, init_right, C,
                       w.ctr + 1);
    BP_HIP(hipGetLastError());
    BP_HIP(hipMemcpyAsync(host, w.ctr, 3 * sizeof(uint32_t), hipMemcpyDeviceToHost, s));
    BP_HIP(hipStreamSynchronize(s));
    if (host[1]) return fail(EKH_EINVAL, "%u neighbour indices outside [0, m = %lld)", host[1], (long long)m);
    if (host[2]) return fail(EKH_EINVAL, "%u starting labels outside [0, %d)", host[2], n_clusters);

    hipLaunchKernelGGL(bp_fill, grid_for(m), dim3(kBs), 0, s, w.deg, m, 0u);
    hipLaunchKernelGGL(bp_degree, grid_for(edges), dim3(kBs), 0, s, nbr, edges, w.deg);
    hipLaunchKernelGGL(bp_fill, grid_for(n), dim3(kBs), 0, s, (uint32_t *)out_left, n, 0xffffffffu); // -1
    hipLaunchKernelGGL(bp_copy_labels, grid_for(m), dim3(kBs), 0, s, init_right, m, out_right);
    BP_HIP(hipGetLastError());
    int32_t rounds = max_rounds;
    for (int32_t rnd = 1; rnd <= max_rounds; ++rnd) {
        hipLaunchKernelGGL(bp_fill, grid_for(C), dim3(kBs), 0, s, w.K_right, C, 0u);
        hipLaunchKernelGGL(bp_fill, grid_for(1), dim3(kBs), 0, s, w.ctr, (int64_t)1, 0u);
        histogram(RightTotals{out_right, w.deg}, m, C, w.K_right, s);
        hipLaunchKernelGGL(bp_left_step, grid_for(n), dim3(kBs), 0, s, nbr, n, k, out_right, w.K_right, two_m, gamma,
                           out_left, w.ctr);
        BP_HIP(hipGetLastError());
        BP_HIP(hipMemcpyAsync(host, w.ctr, sizeof(uint32_t), hipMemcpyDeviceToHost, s));
        BP_HIP(hipStreamSynchronize(s));
        if (host[0] == 0) {
            rounds = rnd;
            break;
        }
        hipLaunchKernelGGL(bp_fill, grid_for(C), dim3(kBs), 0, s, w.cnt_left, C, 0u);
        hipLaunchKernelGGL(bp_fill, grid_for(m * C), dim3(kBs), 0, s, w.counts, m * C, 0u);
        histogram(LeftCounts{out_left}, n, C, w.cnt_left, s);
        hipLaunchKernelGGL(bp_count, grid_for(edges), dim3(kBs), 0, s, nbr, n, k, out_left, C, w.counts);
        hipLaunchKernelGGL(bp_right_step, grid_for(m), dim3(kBs), 0, s, w.counts, m, C, w.deg, w.cnt_left, k, two_m,
                           gamma, out_right);
        BP_HIP(hipGetLastError());
    }
    if (out_rounds) *out_rounds = rounds;
    return EKH_OK;
}

// Edge counts between clusters ("Merges and splits": a single pass of atomic
// adds on the device, whose result the caller reads back once).  Blocks: the range check reads back three
// counters before any count is added.
extern "C" int ekh_cluster_edge_counts(const int32_t *nbr, int64_t n, int32_t k, int64_t m, const int32_t *left,
                                       const int32_t *right, int32_t n_clusters, uint32_t *out_counts, void *ws,
                                       size_t ws_bytes, void *stream) {
    if (!nbr || !left || !right || !out_counts) return fail(EKH_EINVAL, "NULL array");
    if (n < 1 || m < 1) return fail(EKH_EINVAL, "n = %lld and m = %lld must be >= 1", (long long)n, (long long)m);
    if (k < 1 || k > kMaxK) return fail(EKH_EINVAL, "k = %d out of range [1, %d]", k, kMaxK);
    if (n_clusters < 1 || n_clusters > 46340) return fail(EKH_EINVAL, "n_clusters = %d out of range", n_clusters);
    if (n * (int64_t)k >= (int64_t(1) << 31)) return fail(EKH_EINVAL, "n k = %lld edges >= 2^31", (long long)(n * k));
    if (!ws) return fail(EKH_EINVAL, "workspace is NULL");
    if (ws_bytes < 16) return fail(EKH_EWORKSPACE, "workspace %zu bytes < 16 needed", ws_bytes);
    hipStream_t s = (hipStream_t)stream;
    const int64_t edges = n * (int64_t)k, C = n_clusters;
    int64_t span = edges > m ? edges : m;
    span = span > n ? span : n;
    uint32_t *bad = (uint32_t *)ws;
    uint32_t host[3];
    hipLaunchKernelGGL(bp_fill, grid_for(3), dim3(kBs), 0, s, bad, (int64_t)3, 0u);
    hipLaunchKernelGGL(bp_check_labels, grid_for(span), dim3(kBs), 0, s, nbr, edges, m, left, n, right, C, bad);
    BP_HIP(hipGetLastError());
    BP_HIP(hipMemcpyAsync(host, bad, sizeof host, hipMemcpyDeviceToHost, s));
    BP_HIP(hipStreamSynchronize(s));
    if (host[0]) return fail(EKH_EINVAL, "%u neighbour indices outside [0, m = %lld)", host[0], (long long)m);
    if (host[1] || host[2])
        return fail(EKH_EINVAL, "%u left and %u right labels outside [0, %d)", host[1], host[2], n_clusters);
    hipLaunchKernelGGL(bp_fill, grid_for(C * C), dim3(kBs), 0, s, out_counts, C * C, 0u);
    histogram(EdgeBins{nbr, left, right, k, C}, edges, C * C, out_counts, s);
    BP_HIP(hipGetLastError());
    return EKH_OK;
}
