// Greedy k-means++ seeding of libekh (ekh_kmeanspp).
//
// Kilosort4 clustering page, section "The measurement that changed the design:
// serial chains inside a thread": each new seed is the best of 2 + ln k
// candidates drawn by squared distance; the uniforms are made on the host and
// uploaded once, and every draw, score and pick happens on the device with no
// host sync.  The page's lesson is that the candidate scoring must spread over
// many threads: here every point of every candidate has its own thread, and
// the short serial part (pick, weight update, prefix sum, draws) runs in one
// 1024-thread block.  Two launches per seed:
//
//   km_score  grid (point blocks, candidates): squared distance of each point
//             to each candidate, its weight floor(D2 2^S), and per-block sums
//             of min(w, weight) (the candidate's potential, in parts);
//   km_select one block: sums the parts, picks the candidate with the smallest
//             potential, lowers the weights to the new seed, scans them and
//             draws the next seed's candidates.
//
// The arithmetic conventions (float32 distances summed in feature order with
// every operation rounded, weights as exact 64-bit integers, 53-bit uniforms)
// are stated in include/ekh.h; with them every decision is an exact integer
// comparison, independent of the order of any sum.  This file is compiled
// with -ffp-contract=off: no product is fused into a sum.
#include "ekh.h"
#include "host_error.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

namespace {

constexpr int kScoreBs = 256;  // points per score block
constexpr int kSelBs = 1024;   // threads of the select block
constexpr int kSelWaves = kSelBs / 64;
constexpr int kSelR = 4;       // consecutive points per select thread in one pass
constexpr int kMaxCand = 16;
constexpr int kMaxD = 8192;
constexpr int64_t kMaxN = int64_t(1) << 22;
constexpr int32_t kMaxK = 1 << 20;
constexpr int kWeightBits = 40;
constexpr uint64_t kMask53 = (uint64_t(1) << 53) - 1;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return ekh::report_error(code, buf);
}

#define KM_HIP(call)                                                                                                   \
    do {                                                                                                               \
        hipError_t e_ = (call);                                                                                        \
        if (e_ != hipSuccess) return fail(EKH_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));                    \
    } while (0)

// floor(u v / 2^53) for u < 2^53, from the exact 128-bit product
__device__ __forceinline__ uint64_t mul_shift53(uint64_t u, uint64_t v) {
    const uint64_t lo = u * v, hi = __umul64hi(u, v);
    return (hi << 11) | (lo >> 53);
}

__device__ __forceinline__ int64_t first_point(const uint64_t *uniforms, int64_t n) {
    return (int64_t)mul_shift53(uniforms[0] & kMask53, (uint64_t)n);
}

// float32 squared distance of point x to the staged point c, one feature at a
// time in feature order; every subtraction, product and sum rounds to float32
__device__ __forceinline__ float sqdist(const float *__restrict__ X, int64_t ldx, int64_t x, const float *c, int d) {
    float s = 0.0f;
    const float *p = X + x;
    for (int f = 0; f < d; ++f) {
        const float v = p[(int64_t)f * ldx] - c[f];
        const float q = v * v;
        s = s + q;
    }
    return s;
}

// floor(d2 2^S): exact, since the scaling is a power of two and the result
// stays below 2^42
__device__ __forceinline__ uint64_t scaled(float d2, double scale) { return (uint64_t)((double)d2 * scale); }

__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <int BS>
__device__ __forceinline__ uint64_t block_sum(uint64_t v, uint64_t *sh) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 0) sh[wv] = v;
    __syncthreads();
    uint64_t t = 0;
    for (int i = 0; i < BS / 64; ++i) t += sh[i];
    __syncthreads();
    return t;
}

// exclusive prefix of v over the select block; *total receives the block sum
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t v, uint64_t *total, uint64_t *sh) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint64_t inc = v;
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) sh[wv] = inc;
    __syncthreads();
    if (wv == 0) {
        const uint64_t t = lane < kSelWaves ? sh[lane] : 0;
        uint64_t ti = t;
        for (int o = 1; o < kSelWaves; o <<= 1) {
            const uint64_t y = __shfl_up(ti, o);
            if (lane >= o) ti += y;
        }
        if (lane < kSelWaves) sh[lane] = ti - t;
        if (lane == kSelWaves - 1) sh[kSelWaves] = ti;
    }
    __syncthreads();
    *total = sh[kSelWaves];
    const uint64_t r = sh[wv] + inc - v;
    __syncthreads();
    return r;
}

// squared distances to the first seed (point floor(u0 n / 2^53)) and
// per-block maxima
__global__ __launch_bounds__(kScoreBs) void km_first(const float *__restrict__ X, int64_t ldx, int64_t n, int d,
                                                     const uint64_t *uniforms, float *d1, float *bmax) {
    extern __shared__ float cf[];
    __shared__ float wmax[kScoreBs / 64];
    const int64_t first = first_point(uniforms, n);
    for (int f = threadIdx.x; f < d; f += kScoreBs) cf[f] = X[(int64_t)f * ldx + first];
    __syncthreads();
    const int64_t x = (int64_t)blockIdx.x * kScoreBs + threadIdx.x;
    float v = 0.0f;
    if (x < n) {
        v = sqdist(X, ldx, x, cf, d);
        d1[x] = v;
    }
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = wmax[0];
        for (int i = 1; i < kScoreBs / 64; ++i) m = fmaxf(m, wmax[i]);
        bmax[blockIdx.x] = m;
    }
}

// each point against candidate blockIdx.y: its weight to wc, and the block's
// sum of min(w, weight) to partial
__global__ __launch_bounds__(kScoreBs) void km_score(const float *__restrict__ X, int64_t ldx, int64_t n, int d,
                                                     const int32_t *cand, const int32_t *state,
                                                     const uint64_t *__restrict__ w, uint64_t *wc, uint64_t *partial,
                                                     int nb) {
    extern __shared__ float cf[];
    __shared__ uint64_t sh[kScoreBs / 64];
    const int j = blockIdx.y;
    const int64_t c = cand[j];
    for (int f = threadIdx.x; f < d; f += kScoreBs) cf[f] = X[(int64_t)f * ldx + c];
    __syncthreads();
    const double scale = ldexp(1.0, state[0]);
    const int64_t x = (int64_t)blockIdx.x * kScoreBs + threadIdx.x;
    uint64_t m = 0;
    if (x < n) {
        const uint64_t a = scaled(sqdist(X, ldx, x, cf, d), scale);
        wc[j * n + x] = a;
        const uint64_t b = w[x];
        m = a < b ? a : b;
    }
    m = block_sum<kScoreBs>(m, sh);
    if (threadIdx.x == 0) partial[(int64_t)j * nb + blockIdx.x] = m;
}

// s == 0: weights from the first seed (S from the largest squared distance);
// s >= 1: seed s is the candidate with the smallest potential (first drawn on
// ties), and the weights drop to it.  Unless s is the last seed, the L
// candidates of seed s + 1 are then drawn from uniforms 1 + s L + j.
__global__ __launch_bounds__(kSelBs) void km_select(int s, int k, int L, int64_t n, int nb, const uint64_t *uniforms,
                                                    const float *d1, const float *bmax, const uint64_t *partial,
                                                    const uint64_t *wc, uint64_t *w, int32_t *cand, int32_t *state,
                                                    int32_t *seeds, int64_t *out_potential) {
    __shared__ uint64_t sh[kSelWaves + 1];
    __shared__ uint64_t phi[kMaxCand];
    __shared__ uint64_t thr[kMaxCand];
    __shared__ int32_t pick[kMaxCand];
    __shared__ float smax[kSelWaves];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const bool init = s == 0;
    double scale = 1.0;
    int jb = 0;
    uint64_t T;
    if (init) {
        float mx = 0.0f;
        for (int b = tid; b < nb; b += kSelBs) mx = fmaxf(mx, bmax[b]);
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        if (lane == 0) smax[wv] = mx;
        __syncthreads();
        mx = smax[0];
        for (int i = 1; i < kSelWaves; ++i) mx = fmaxf(mx, smax[i]);
        int S = 0;
        if (mx > 0.0f) {
            int e;
            frexpf(mx, &e); // mx = m 2^e, 0.5 <= m < 1
            S = kWeightBits - e;
        }
        scale = ldexp(1.0, S);
        uint64_t loc = 0;
        for (int64_t x = tid; x < n; x += kSelBs) loc += scaled(d1[x], scale);
        T = block_sum<kSelBs>(loc, sh);
        if (tid == 0) {
            state[0] = S;
            seeds[0] = (int32_t)first_point(uniforms, n);
        }
    } else {
        if (wv < L) {
            uint64_t a = 0;
            for (int b = lane; b < nb; b += 64) a += partial[(int64_t)wv * nb + b];
            a = wave_sum(a);
            if (lane == 0) phi[wv] = a;
        }
        __syncthreads();
        for (int j = 1; j < L; ++j)
            if (phi[j] < phi[jb]) jb = j;
        T = phi[jb];
        if (tid == 0) seeds[s] = cand[jb];
    }
    if (s == k - 1) {
        if (tid == 0 && out_potential) *out_potential = (int64_t)T;
        return;
    }
    if (tid < L) {
        thr[tid] = mul_shift53(uniforms[1 + (int64_t)s * L + tid] & kMask53, T);
        pick[tid] = 0;
    }
    __syncthreads();
    const uint64_t *wj = wc + (int64_t)jb * n;
    uint64_t carry = 0;
    for (int64_t base = 0; base < n; base += (int64_t)kSelBs * kSelR) {
        const int64_t x0 = base + (int64_t)tid * kSelR;
        uint64_t v[kSelR], loc = 0;
#pragma unroll
        for (int r = 0; r < kSelR; ++r) {
            const int64_t x = x0 + r;
            uint64_t a = 0;
            if (x < n) {
                if (init) {
                    a = scaled(d1[x], scale);
                } else {
                    const uint64_t p = w[x], q = wj[x];
                    a = p < q ? p : q;
                }
                w[x] = a;
            }
            v[r] = a;
            loc += a;
        }
        uint64_t tot;
        uint64_t p = carry + block_excl_scan(loc, &tot, sh);
#pragma unroll
        for (int r = 0; r < kSelR; ++r) {
            const uint64_t q = p + v[r];
            if (v[r])
                for (int j = 0; j < L; ++j)
                    if (p <= thr[j] && thr[j] < q) pick[j] = (int32_t)(x0 + r);
            p = q;
        }
        carry += tot;
    }
    __syncthreads();
    if (tid < L) cand[tid] = pick[tid];
}

struct Ws {
    uint64_t *w, *wc, *partial;
    float *d1, *bmax;
    int32_t *cand, *state;
    size_t bytes;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int n_candidates(int32_t k) { return k > 1 ? 2 + (int)std::floor(std::log((double)k)) : 0; }

Ws carve(void *base, int64_t n, int L) {
    Ws ws{};
    char *p = (char *)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        void *q = p ? (void *)(p + off) : nullptr;
        off += align256(bytes);
        return q;
    };
    const int64_t nb = (n + kScoreBs - 1) / kScoreBs;
    const int Lw = L > 1 ? L : 1;
    ws.w = (uint64_t *)take(n * 8);
    ws.wc = (uint64_t *)take((size_t)Lw * n * 8);
    ws.partial = (uint64_t *)take((size_t)Lw * nb * 8);
    ws.d1 = (float *)take(n * 4);
    ws.bmax = (float *)take(nb * 4);
    ws.cand = (int32_t *)take(kMaxCand * 4);
    ws.state = (int32_t *)take(16);
    ws.bytes = off;
    return ws;
}

} // namespace

extern "C" size_t ekh_kmeanspp_workspace_bytes(int64_t n, int32_t k) {
    if (n < 1 || n > kMaxN || k < 1 || k > kMaxK) return 0;
    return carve(nullptr, n, n_candidates(k)).bytes;
}

extern "C" int ekh_kmeanspp(const float *X, int64_t ldx, int64_t n, int32_t d, int32_t k, const uint64_t *uniforms,
                            int64_t n_uniforms, int32_t *out_seeds, int64_t *out_potential, void *ws, size_t ws_bytes,
                            void *stream) {
    if (!X || !uniforms || !out_seeds) return fail(EKH_EINVAL, "NULL array");
    if (n < 1 || n > kMaxN) return fail(EKH_EINVAL, "n = %lld out of range [1, 2^22]", (long long)n);
    if (d < 1 || d > kMaxD) return fail(EKH_EINVAL, "d = %d out of range [1, %d]", d, kMaxD);
    if (ldx < n) return fail(EKH_EINVAL, "ldx = %lld < n = %lld", (long long)ldx, (long long)n);
    if (k < 1 || k > kMaxK) return fail(EKH_EINVAL, "k = %d out of range [1, 2^20]", k);
    const int L = n_candidates(k);
    const int64_t need = 1 + (int64_t)(k - 1) * L;
    if (n_uniforms < need)
        return fail(EKH_EINVAL, "%lld uniforms given, %lld needed (1 + (k - 1) L, L = %d)", (long long)n_uniforms,
                    (long long)need, L);
    if (!ws) return fail(EKH_EINVAL, "workspace is NULL");
    const Ws w = carve(ws, n, L);
    if (ws_bytes < w.bytes) return fail(EKH_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.bytes);
    hipStream_t st = (hipStream_t)stream;
    const int nb = (int)((n + kScoreBs - 1) / kScoreBs);
    const size_t lds = (size_t)d * sizeof(float);
    hipLaunchKernelGGL(km_first, dim3(nb), dim3(kScoreBs), lds, st, X, ldx, n, d, uniforms, w.d1, w.bmax);
    hipLaunchKernelGGL(km_select, dim3(1), dim3(kSelBs), 0, st, 0, k, L, n, nb, uniforms, w.d1, w.bmax, w.partial,
                       w.wc, w.w, w.cand, w.state, out_seeds, out_potential);
    KM_HIP(hipGetLastError());
    for (int s = 1; s < k; ++s) {
        hipLaunchKernelGGL(km_score, dim3(nb, L), dim3(kScoreBs), lds, st, X, ldx, n, d, w.cand, w.state, w.w, w.wc,
                           w.partial, nb);
        hipLaunchKernelGGL(km_select, dim3(1), dim3(kSelBs), 0, st, s, k, L, n, nb, uniforms, w.d1, w.bmax,
                           w.partial, w.wc, w.w, w.cand, w.state, out_seeds, out_potential);
    }
    KM_HIP(hipGetLastError());
    return EKH_OK;
}
