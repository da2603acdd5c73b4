// Greedy k-means++ seeding of libekh (ekh_kmeanspp).
//
// Kilosort4 clustering page, section "The measurement that changed the design:
// serial chains inside a thread".  The method there: after the first seed,
// 2 + ln k candidates are sampled with weights given by their squared distance
// to the nearest seed so far, and the one that leaves the lowest potential is
// kept.  The random numbers come from the host in one upload, and the device
// does all sampling, scoring and picking without waiting on the host.  The page's lesson is that no thread may carry a long serial
// chain.  Seeding is one chain of k dependent steps, each short (sum L
// candidates' potentials, pick, lower the weights, scan, draw), so what
// matters is how little latency each step costs.  Two paths, same results:
//
//  * small sections (n <= 4096 and n at most 4 times the candidate draws):
//    km_dist_matrix computes every pairwise squared distance at once over the
//    whole chip (the same float32 arithmetic, in the same feature order), then
//    km_seed_block, one 1024-thread block, runs all k seeds with the weights
//    in registers: per seed one block scan, one gather of the L candidates'
//    rows and one block reduction, with no launch in between;
//  * larger sections, two launches per seed:
//      km_score  grid (point blocks, candidates): squared distance of each
//                point to each candidate, its weight floor(D2 2^S), and
//                per-block sums of min(w, weight) (the potential, in parts);
//      km_select one block: sums the parts, picks the candidate with the
//                smallest potential, lowers the weights, scans them and draws
//                the next seed's candidates.
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

constexpr int kScoreBs = 64;  // points per score block
constexpr int kSelBs = 1024;   // threads of the select block
constexpr int kSelWaves = kSelBs / 64;
constexpr int kSelR = 4;       // consecutive points per select thread in one pass
constexpr int kMaxCand = 16;
constexpr int kMaxD = 8192;
constexpr int64_t kMaxN = int64_t(1) << 22;
constexpr int32_t kMaxK = 1 << 20;
constexpr int kWeightBits = 40;
constexpr uint64_t kMask53 = (uint64_t(1) << 53) - 1;
constexpr int kMatX = 256;            // columns (points) per distance-matrix block
constexpr int kMatR = 16;             // rows per distance-matrix block
constexpr int kMatF = 128;            // features staged per pass of a matrix block
constexpr int kSeedR = 4;             // points per thread of the seeding block
constexpr int kBlockMaxN = kSelBs * kSeedR;
constexpr int kRingSeeds = 64;        // seeds whose uniforms the seeding block holds in LDS
constexpr int kBlockMaxL = 7;         // candidates per seed the seeding block keeps in registers (k <= 403)
constexpr int kBlockMaxK = 403;       // the largest k with L <= 7
static_assert(kMaxCand <= kSelWaves, "one wave per candidate sums the potentials");

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

// floor(d2 2^S) from the bits of d2 >= 0: with d2 = m 2^(e - 150) (m the
// 24-bit significand, e the biased exponent; e = 1 for subnormals) the result
// is m shifted by e - 150 + S, exact.  For finite inputs it stays below 2^43;
// both shifts are clamped (and selected without a branch) so that no input
// makes one undefined.
__device__ __forceinline__ uint64_t scaled(float d2, int S) {
    const uint32_t b = __float_as_uint(d2);
    const int e = (int)(b >> 23);
    const uint64_t m = (b & 0x7fffffu) | (e ? 0x800000u : 0u);
    const int sh = (e ? e : 1) - 150 + S;
    const uint64_t up = m << (sh < 0 ? 0 : sh < 39 ? sh : 39);
    const uint64_t down = m >> (sh > 0 ? 0 : -sh < 63 ? -sh : 63);
    return sh >= 0 ? up : down;
}

// S = 40 - e for the largest squared distance m 2^e (0.5 <= m < 1) to the
// first seed, 0 when all are 0: every weight then stays below 2^40
__device__ __forceinline__ int scale_exponent(float mx) {
    if (!(mx > 0.0f)) return 0;
    int e;
    frexpf(mx, &e);
    return kWeightBits - e;
}

__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// L independent wave sums, one butterfly step for all of them at a time (the
// shuffles of a step are in flight together)
template <int L>
__device__ __forceinline__ void wave_sums(uint64_t (&m)[L]) {
    for (int o = 32; o > 0; o >>= 1) {
        uint64_t t[L];
#pragma unroll
        for (int j = 0; j < L; ++j) t[j] = __shfl_xor(m[j], o);
#pragma unroll
        for (int j = 0; j < L; ++j) m[j] += t[j];
    }
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

// exclusive prefix of v over a block of nw waves; *total receives the block sum
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t v, uint64_t *total, uint64_t *sh, int nw) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint64_t inc = v;
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) sh[wv] = inc;
    __syncthreads();
    if (wv == 0) {
        const uint64_t t = lane < nw ? sh[lane] : 0;
        uint64_t ti = t;
        for (int o = 1; o < nw; o <<= 1) {
            const uint64_t y = __shfl_up(ti, o);
            if (lane >= o) ti += y;
        }
        if (lane < nw) sh[lane] = ti - t;
        if (lane == nw - 1) sh[kSelWaves] = ti;
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
    const int S = state[0];
    const int64_t x = (int64_t)blockIdx.x * kScoreBs + threadIdx.x;
    uint64_t m = 0;
    if (x < n) {
        const uint64_t a = scaled(sqdist(X, ldx, x, cf, d), S);
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
    int S = 0;
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
        S = scale_exponent(mx);
        uint64_t loc = 0;
        for (int64_t x = tid; x < n; x += kSelBs) loc += scaled(d1[x], S);
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
                    a = scaled(d1[x], S);
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
        uint64_t p = carry + block_excl_scan(loc, &tot, sh, kSelWaves);
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

// D[c * ldD + x] = squared distance of points c and x with the arithmetic of
// sqdist (feature order, every operation rounded; symmetric bit for bit).  A
// block: kMatR rows against kMatX columns, the rows' features staged in LDS.
__global__ __launch_bounds__(kMatX) void km_dist_matrix(const float *__restrict__ X, int64_t ldx, int n, int d,
                                                        int ldD, float *D) {
    __shared__ float cs[kMatF][kMatR];
    const int x = blockIdx.x * kMatX + threadIdx.x;
    const int c0 = blockIdx.y * kMatR;
    const float *px = X + (x < n ? x : n - 1);
    float s[kMatR];
#pragma unroll
    for (int r = 0; r < kMatR; ++r) s[r] = 0.0f;
    for (int f0 = 0; f0 < d; f0 += kMatF) {
        const int fc = d - f0 < kMatF ? d - f0 : kMatF;
        __syncthreads();
        for (int i = threadIdx.x; i < fc * kMatR; i += kMatX) {
            const int f = i / kMatR, r = i % kMatR, c = c0 + r < n ? c0 + r : n - 1;
            cs[f][r] = X[(int64_t)(f0 + f) * ldx + c];
        }
        __syncthreads();
#pragma unroll 4
        for (int f = 0; f < fc; ++f) {
            const float xv = px[(int64_t)(f0 + f) * ldx];
#pragma unroll
            for (int r = 0; r < kMatR; ++r) {
                const float v = xv - cs[f][r];
                const float q = v * v;
                s[r] = s[r] + q;
            }
        }
    }
    if (x < n)
#pragma unroll
        for (int r = 0; r < kMatR; ++r)
            if (c0 + r < n) D[(int64_t)(c0 + r) * ldD + x] = s[r];
}

// All k seeds in one block from the distance matrix (rows of stride ldD, a
// multiple of 4).  The block has 64 ceil(n / 256) threads; thread t owns
// points 4t .. 4t+3 and keeps, per point, the squared distance to its nearest
// seed (dn) and its weight w = floor(dn 2^S).  A candidate's potential is
// T - gain with gain = sum of w - floor(d 2^S) over the points it is closer
// to (min(w, floor(d 2^S)) = w - max(0, w - floor(d 2^S)), and the floor is
// monotone), so only the captured points need the conversion.  Per seed:
// thresholds from T, a block scan that locates the L draws, a float4 gather
// of the L candidates' rows for the thread's points, a block reduction of the
// L gains, the pick (smallest potential, first drawn on ties) and the update.
template <int L>
__global__ __launch_bounds__(kSelBs) void km_seed_block(const float *__restrict__ D, int n, int ldD, int k,
                                                        const uint64_t *uniforms, int32_t *seeds,
                                                        int64_t *out_potential) {
    __shared__ uint64_t sh[kSelWaves + 1];
    __shared__ uint64_t part[kSelWaves][L];
    __shared__ uint64_t phi[L];
    __shared__ uint64_t thr[L];
    __shared__ int32_t pick[L];
    __shared__ float smax[kSelWaves];
    __shared__ uint64_t uring[kRingSeeds * L]; // the uniforms of the next kRingSeeds seeds
    __shared__ int32_t chosen[kBlockMaxK];      // the seeds, written out at the end (a global store
                                                // inside the loop would hold up the next barrier)
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = (int)(blockDim.x >> 6);
    const int x0 = tid * kSeedR;
    const bool has = x0 < n;
    const int first = (int)first_point(uniforms, n);
    float4 d1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (has) d1 = *(const float4 *)(D + (int64_t)first * ldD + x0);
    float dn[kSeedR];
    float mx = 0.0f;
#pragma unroll
    for (int r = 0; r < kSeedR; ++r) {
        dn[r] = x0 + r < n ? (&d1.x)[r] : -INFINITY; // no distance is below -inf: padding never counts
        mx = fmaxf(mx, dn[r]);
    }
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) smax[wv] = mx;
    __syncthreads();
    mx = smax[0];
    for (int i = 1; i < nw; ++i) mx = fmaxf(mx, smax[i]);
    const int S = scale_exponent(mx);
    uint64_t w[kSeedR], loc = 0;
#pragma unroll
    for (int r = 0; r < kSeedR; ++r) {
        w[r] = x0 + r < n ? scaled(dn[r], S) : 0;
        loc += w[r];
    }
    uint64_t T = wave_sum(loc);
    if (lane == 0) sh[wv] = T;
    __syncthreads();
    T = 0;
    for (int i = 0; i < nw; ++i) T += sh[i];
    if (tid == 0) chosen[0] = first;
    for (int s = 1; s < k; ++s) {
        const int slot = (s - 1) % kRingSeeds;
        if (slot == 0) { // refill the ring: seeds s .. s + kRingSeeds - 1 (one memory round trip per refill)
            const int64_t base = 1 + (int64_t)(s - 1) * L, end = 1 + (int64_t)(k - 1) * L;
            for (int i = tid; i < kRingSeeds * L; i += blockDim.x)
                uring[i] = base + i < end ? uniforms[base + i] & kMask53 : 0;
        }
        __syncthreads(); // the ring is filled; every read of sh, phi and pick of the previous seed is done
        if (tid < L) {
            thr[tid] = mul_shift53(uring[slot * L + tid], T);
            pick[tid] = 0;
        }
        __syncthreads();
        uint64_t th[L];
#pragma unroll
        for (int j = 0; j < L; ++j) th[j] = thr[j];
        uint64_t tot;
        uint64_t p = block_excl_scan(loc, &tot, sh, nw);
#pragma unroll
        for (int r = 0; r < kSeedR; ++r) {
            const uint64_t q = p + w[r];
#pragma unroll
            for (int j = 0; j < L; ++j)
                if (p <= th[j] && th[j] < q) pick[j] = x0 + r; // empty ranges (w = 0) never match
            p = q;
        }
        __syncthreads();
        int32_t cj[L];
#pragma unroll
        for (int j = 0; j < L; ++j) cj[j] = pick[j];
        float4 dv[L];
#pragma unroll
        for (int j = 0; j < L; ++j)
            dv[j] = has ? *(const float4 *)(D + (int64_t)cj[j] * ldD + x0) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        uint64_t g[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            g[j] = 0;
#pragma unroll
            for (int r = 0; r < kSeedR; ++r) {
                const float d = (&dv[j].x)[r];
                if (d < dn[r]) g[j] += w[r] - scaled(d, S);
            }
        }
        wave_sums<L>(g);
        if (lane == 0)
#pragma unroll
            for (int j = 0; j < L; ++j) part[wv][j] = g[j];
        __syncthreads();
        if (tid < L) {
            uint64_t a = 0;
            for (int i = 0; i < nw; ++i) a += part[i][tid];
            phi[tid] = T - a;
        }
        __syncthreads();
        int jb = 0;
        uint64_t best = phi[0];
#pragma unroll
        for (int j = 1; j < L; ++j) {
            const uint64_t v = phi[j];
            if (v < best) {
                best = v;
                jb = j;
            }
        }
        T = best;
        int32_t cb = cj[0];
        float4 db = dv[0];
#pragma unroll
        for (int j = 1; j < L; ++j)
            if (j == jb) {
                cb = cj[j];
                db = dv[j];
            }
        if (tid == 0) chosen[s] = cb;
        loc = 0;
#pragma unroll
        for (int r = 0; r < kSeedR; ++r) {
            const float d = (&db.x)[r];
            if (d < dn[r]) {
                dn[r] = d;
                w[r] = scaled(d, S);
            }
            loc += w[r];
        }
    }
    __syncthreads();
    for (int i = tid; i < k; i += blockDim.x) seeds[i] = chosen[i];
    if (tid == 0 && out_potential) *out_potential = (int64_t)T;
}

template <int L>
void launch_seed_block(const float *D, int n, int ldD, int k, const uint64_t *uniforms, int32_t *seeds, int64_t *pot,
                       hipStream_t st) {
    const unsigned threads = 64u * (unsigned)((n + 64 * kSeedR - 1) / (64 * kSeedR));
    hipLaunchKernelGGL(km_seed_block<L>, dim3(1), dim3(threads), 0, st, D, n, ldD, k, uniforms, seeds, pot);
}

bool seed_block_dispatch(int L, const float *D, int n, int ldD, int k, const uint64_t *uniforms, int32_t *seeds,
                         int64_t *pot, hipStream_t st) {
    switch (L) {
    case 2: launch_seed_block<2>(D, n, ldD, k, uniforms, seeds, pot, st); return true;
    case 3: launch_seed_block<3>(D, n, ldD, k, uniforms, seeds, pot, st); return true;
    case 4: launch_seed_block<4>(D, n, ldD, k, uniforms, seeds, pot, st); return true;
    case 5: launch_seed_block<5>(D, n, ldD, k, uniforms, seeds, pot, st); return true;
    case 6: launch_seed_block<6>(D, n, ldD, k, uniforms, seeds, pot, st); return true;
    case 7: launch_seed_block<7>(D, n, ldD, k, uniforms, seeds, pot, st); return true;
    default: return false;
    }
}

struct Ws {
    uint64_t *w, *wc, *partial;
    float *d1, *bmax, *D;
    int32_t *cand, *state;
    size_t bytes;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int n_candidates(int32_t k) { return k > 1 ? 2 + (int)std::floor(std::log((double)k)) : 0; }

// the distance-matrix path: sections small enough for one block's registers
// (n <= 4096, L <= 7, i.e. k <= 403), with enough draws (at least n / 4
// candidate rows) that computing every row costs no more than a few times the
// rows the seeding reads
bool use_block(int64_t n, int32_t k, int L, uint32_t flags) {
    return !(flags & EKH_KMEANSPP_PER_SEED_LAUNCHES) && n <= kBlockMaxN && L >= 2 && L <= kBlockMaxL && k <= kBlockMaxK &&
           n <= 4 * (1 + (int64_t)(k - 1) * L);
}

Ws carve(void *base, int64_t n, int L, bool block) {
    Ws ws{};
    char *p = (char *)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        void *q = p ? (void *)(p + off) : nullptr;
        off += align256(bytes);
        return q;
    };
    if (block) {
        ws.D = (float *)take((size_t)n * (size_t)((n + 3) / 4 * 4) * 4);
    } else {
        const int64_t nb = (n + kScoreBs - 1) / kScoreBs;
        const int Lw = L > 1 ? L : 1;
        ws.w = (uint64_t *)take(n * 8);
        ws.wc = (uint64_t *)take((size_t)Lw * n * 8);
        ws.partial = (uint64_t *)take((size_t)Lw * nb * 8);
        ws.d1 = (float *)take(n * 4);
        ws.bmax = (float *)take(nb * 4);
        ws.cand = (int32_t *)take(kMaxCand * 4);
        ws.state = (int32_t *)take(16);
    }
    ws.bytes = off;
    return ws;
}

} // namespace

extern "C" size_t ekh_kmeanspp_workspace_bytes(int64_t n, int32_t k, uint32_t flags) {
    if (n < 1 || n > kMaxN || k < 1 || k > kMaxK || (flags & ~EKH_KMEANSPP_PER_SEED_LAUNCHES)) return 0;
    const int L = n_candidates(k);
    return carve(nullptr, n, L, use_block(n, k, L, flags)).bytes;
}

extern "C" int ekh_kmeanspp(const float *X, int64_t ldx, int64_t n, int32_t d, int32_t k, const uint64_t *uniforms,
                            int64_t n_uniforms, uint32_t flags, int32_t *out_seeds, int64_t *out_potential, void *ws,
                            size_t ws_bytes, void *stream) {
    if (!X || !uniforms || !out_seeds) return fail(EKH_EINVAL, "NULL array");
    if (n < 1 || n > kMaxN) return fail(EKH_EINVAL, "n = %lld out of range [1, 2^22]", (long long)n);
    if (d < 1 || d > kMaxD) return fail(EKH_EINVAL, "d = %d out of range [1, %d]", d, kMaxD);
    if (ldx < n || ldx >= (int64_t(1) << 25))
        return fail(EKH_EINVAL, "ldx = %lld outside [n = %lld, 2^25)", (long long)ldx, (long long)n);
    if (k < 1 || k > kMaxK) return fail(EKH_EINVAL, "k = %d out of range [1, 2^20]", k);
    if (flags & ~EKH_KMEANSPP_PER_SEED_LAUNCHES) return fail(EKH_EINVAL, "unknown flags 0x%x", flags);
    const int L = n_candidates(k);
    const int64_t need = 1 + (int64_t)(k - 1) * L;
    if (n_uniforms < need)
        return fail(EKH_EINVAL, "%lld uniforms given, %lld needed (1 + (k - 1) L, L = %d)", (long long)n_uniforms,
                    (long long)need, L);
    if (!ws) return fail(EKH_EINVAL, "workspace is NULL");
    const bool block = use_block(n, k, L, flags);
    const Ws w = carve(ws, n, L, block);
    if (ws_bytes < w.bytes) return fail(EKH_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.bytes);
    hipStream_t st = (hipStream_t)stream;
    if (block) {
        const dim3 grid((unsigned)((n + kMatX - 1) / kMatX), (unsigned)((n + kMatR - 1) / kMatR));
        const int ldD = (int)((n + 3) / 4 * 4);
        hipLaunchKernelGGL(km_dist_matrix, grid, dim3(kMatX), 0, st, X, ldx, (int)n, d, ldD, w.D);
        if (!seed_block_dispatch(L, w.D, (int)n, ldD, k, uniforms, out_seeds, out_potential, st))
            return fail(EKH_EINTERNAL, "no seeding block for L = %d", L);
        KM_HIP(hipGetLastError());
        return EKH_OK;
    }
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
