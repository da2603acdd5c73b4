// Host HDBSCAN tail of libekh: spanning tree -> single-linkage hierarchy ->
// condensed tree -> excess-of-mass selection -> labels (ekh_hdbscan_tail).
//
// The HDBSCAN page ("The algorithm on the device", last item) runs these
// steps on the host, in linear time, after the device has built the tree; the
// same section fixes the edge order (weight, lower index, higher index).  The
// steps themselves are the standard HDBSCAN* definitions; the conventions that
// make the result exactly reproducible (merge order of equal weights, cluster
// numbering, summation order of the stabilities, the excess-of-mass tie) are
// stated in include/ekh.h.
//
// Plain C++ (no device code): union-find over the n - 1 edges, one top-down
// walk of the hierarchy that emits every point once, a breadth-first
// renumbering of the clusters, then two passes over the clusters.  O(n log n)
// for the final ordering of the condensed tree, O(n) otherwise.
#include "ekh.h"
#include "host_error.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <numeric>
#include <vector>

namespace {

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return ekh::report_error(code, buf);
}

// lambda = 1 / w, +inf for w = 0 (w is a float32 weight, widened exactly)
inline double lambda_of(float w) {
    return w == 0.f ? std::numeric_limits<double>::infinity() : 1.0 / (double)w;
}

struct Entry {
    int64_t parent, child;
    double lambda;
    int64_t size;
};

// Stable LSD radix sort of (key, value) pairs by key, 11-bit digits over the
// key bits in use.
void radix_sort(std::vector<uint64_t> &key, std::vector<uint32_t> &val) {
    const size_t m = key.size();
    uint64_t any = 0;
    for (const uint64_t k : key) any |= k;
    int bits = 0;
    while (bits < 64 && (any >> bits)) ++bits;
    std::vector<uint64_t> k2(m);
    std::vector<uint32_t> v2(m);
    std::vector<size_t> cnt(2049);
    for (int sh = 0; sh < bits; sh += 11) {
        std::fill(cnt.begin(), cnt.end(), 0);
        for (size_t i = 0; i < m; ++i) ++cnt[((key[i] >> sh) & 2047) + 1];
        for (int b = 0; b < 2048; ++b) cnt[b + 1] += cnt[b];
        for (size_t i = 0; i < m; ++i) {
            const size_t d = cnt[(key[i] >> sh) & 2047]++;
            k2[d] = key[i];
            v2[d] = val[i];
        }
        key.swap(k2);
        val.swap(v2);
    }
}

struct Tail {
    int64_t n;
    int64_t mcs;
    // hierarchy: internal node n + k (k = 0 .. n - 2) merges left[k] and right[k] at dist[k]
    // (32-bit: node ids stay below 2n <= 2^31)
    std::vector<int32_t> left, right, size, minpt;
    std::vector<float> dist;
    // provisional clusters (creation order), then final ids n + c
    std::vector<double> birth;
    std::vector<int64_t> first_min, kid0, kid1, parent;
    std::vector<Entry> raw; // parent / child clusters provisional here
    std::vector<char> child_is_cluster;

    int build_hierarchy(const int32_t *lo, const int32_t *hi, const float *w) {
        const int64_t m = n - 1;
        for (int64_t e = 0; e < m; ++e) {
            if (lo[e] < 0 || hi[e] >= n || lo[e] >= hi[e])
                return fail(EKH_EINVAL, "edge %lld: (%d, %d) needs 0 <= lo < hi < n = %lld", (long long)e, lo[e],
                            hi[e], (long long)n);
            if (!(w[e] >= 0.f) || std::isinf(w[e]))
                return fail(EKH_EINVAL, "edge %lld: weight %g is not finite and >= 0", (long long)e, (double)w[e]);
        }
        auto less = [&](int64_t a, int64_t b) {
            if (w[a] != w[b]) return w[a] < w[b];
            if (lo[a] != lo[b]) return lo[a] < lo[b];
            return hi[a] < hi[b];
        };
        std::vector<int64_t> order(m);
        std::iota(order.begin(), order.end(), int64_t(0));
        bool sorted = true;
        for (int64_t e = 0; e + 1 < m && sorted; ++e) sorted = !less(e + 1, e);
        if (!sorted) std::stable_sort(order.begin(), order.end(), less);

        std::vector<int32_t> uf(n), ufsize(n, 1), top(n);
        std::iota(uf.begin(), uf.end(), int32_t(0));
        std::iota(top.begin(), top.end(), int32_t(0));
        auto find = [&](int32_t x) {
            while (uf[x] != x) {
                uf[x] = uf[uf[x]];
                x = uf[x];
            }
            return x;
        };
        left.resize(m);
        right.resize(m);
        dist.resize(m);
        size.assign(2 * n - 1, 1);
        minpt.resize(2 * n - 1);
        std::iota(minpt.begin(), minpt.begin() + n, int32_t(0));
        for (int64_t k = 0; k < m; ++k) {
            const int64_t e = order[k];
            int32_t ra = find(lo[e]), rb = find(hi[e]);
            if (ra == rb) return fail(EKH_EINVAL, "edges do not form a spanning tree (cycle at edge %lld)", (long long)e);
            const int32_t node = (int32_t)(n + k), a = top[ra], b = top[rb];
            left[k] = a;
            right[k] = b;
            dist[k] = w[e];
            size[node] = size[a] + size[b];
            minpt[node] = std::min(minpt[a], minpt[b]);
            if (ufsize[ra] < ufsize[rb]) std::swap(ra, rb);
            uf[rb] = ra;
            ufsize[ra] += ufsize[rb];
            top[ra] = node;
        }
        return EKH_OK;
    }

    int64_t new_cluster(double b, int64_t fm, int64_t par) {
        birth.push_back(b);
        first_min.push_back(fm);
        kid0.push_back(-1);
        kid1.push_back(-1);
        parent.push_back(par);
        return (int64_t)birth.size() - 1;
    }

    // every point below `node` leaves cluster c at lambda
    void emit_points(int64_t node, int64_t c, double lam, std::vector<int64_t> &stack) {
        stack.clear();
        stack.push_back(node);
        while (!stack.empty()) {
            const int64_t x = stack.back();
            stack.pop_back();
            if (x < n) {
                raw.push_back(Entry{c, x, lam, 1});
                child_is_cluster.push_back(0);
            } else {
                stack.push_back(left[x - n]);
                stack.push_back(right[x - n]);
            }
        }
    }

    void condense() {
        raw.reserve(n + 2 * (n / mcs) + 2);
        child_is_cluster.reserve(raw.capacity());
        const int64_t topnode = 2 * n - 2;
        new_cluster(0.0, minpt[topnode], -1);
        std::vector<std::pair<int64_t, int64_t>> work{{topnode, 0}};
        std::vector<int64_t> stack;
        while (!work.empty()) {
            int64_t node = work.back().first;
            const int64_t c = work.back().second;
            work.pop_back();
            for (;;) {
                const int64_t k = node - n, a = left[k], b = right[k];
                const double lam = lambda_of(dist[k]);
                const bool la = size[a] >= mcs, lb = size[b] >= mcs;
                if (la && lb) {
                    for (const int64_t ch : {a, b}) {
                        const int64_t pc = new_cluster(lam, minpt[ch], c);
                        (kid0[c] < 0 ? kid0[c] : kid1[c]) = pc;
                        raw.push_back(Entry{c, pc, lam, size[ch]});
                        child_is_cluster.push_back(1);
                        work.emplace_back(ch, pc);
                    }
                    break;
                }
                if (la || lb) {
                    emit_points(la ? b : a, c, lam, stack);
                    node = la ? a : b;
                    continue;
                }
                emit_points(a, c, lam, stack);
                emit_points(b, c, lam, stack);
                break;
            }
        }
    }
};

} // namespace

extern "C" int ekh_hdbscan_tail(const int32_t *lo, const int32_t *hi, const float *w, int64_t n,
                                int32_t min_cluster_size, int32_t *out_labels, int64_t *ct_parent, int64_t *ct_child,
                                double *ct_lambda, int64_t *ct_size, double *out_stability, ekh_hdbscan_info *info) {
    if (n < 1 || n > (int64_t(1) << 30)) return fail(EKH_EINVAL, "n = %lld out of range [1, 2^30]", (long long)n);
    if (min_cluster_size < 2) return fail(EKH_EINVAL, "min_cluster_size = %d must be >= 2", min_cluster_size);
    if (!out_labels) return fail(EKH_EINVAL, "out_labels is NULL");
    if (n > 1 && (!lo || !hi || !w)) return fail(EKH_EINVAL, "edge arrays must not be NULL");
    const bool want_tree = ct_parent || ct_child || ct_lambda || ct_size;
    if (want_tree && !(ct_parent && ct_child && ct_lambda && ct_size))
        return fail(EKH_EINVAL, "the four condensed-tree arrays are given together or not at all");

    if (n == 1) {
        out_labels[0] = -1;
        if (out_stability) out_stability[0] = 0.0;
        if (info) *info = ekh_hdbscan_info{0, 1, 0};
        return EKH_OK;
    }
    Tail T;
    T.n = n;
    T.mcs = min_cluster_size;
    if (int rc = T.build_hierarchy(lo, hi, w)) return rc;
    T.condense();

    // breadth-first ids: root n; the two children of a split by ascending smallest point
    const int64_t ncl = (int64_t)T.birth.size();
    std::vector<int64_t> fid(ncl), by_id(ncl);
    fid[0] = n;
    by_id[0] = 0;
    int64_t next = 1;
    for (int64_t q = 0; q < next; ++q) {
        const int64_t c = by_id[q];
        if (T.kid0[c] < 0) continue;
        int64_t k0 = T.kid0[c], k1 = T.kid1[c];
        if (T.first_min[k1] < T.first_min[k0]) std::swap(k0, k1);
        fid[k0] = n + next;
        by_id[next++] = k0;
        fid[k1] = n + next;
        by_id[next++] = k1;
    }

    // entries in ascending (parent, child) order: a radix sort of the packed
    // key (parent - n) << cb | child, cb = the bits of the largest child id
    // (children are below n + clusters < 2^31; the pairs are distinct)
    const int64_t ne = (int64_t)T.raw.size();
    int cb = 0;
    while ((int64_t(1) << cb) < n + ncl) ++cb;
    const uint64_t cmask = (uint64_t(1) << cb) - 1;
    std::vector<uint64_t> key(ne);
    std::vector<uint32_t> at(ne);
    for (int64_t i = 0; i < ne; ++i) {
        const Entry &r = T.raw[i];
        const uint64_t child = (uint64_t)(T.child_is_cluster[i] ? fid[r.child] : r.child);
        key[i] = (uint64_t)(fid[r.parent] - n) << cb | child;
        at[i] = (uint32_t)i;
    }
    radix_sort(key, at);
    // entry j of the sorted list: parent n + (key[j] >> cb), child key[j] & cmask,
    // lambda and size from T.raw[at[j]]

    // stabilities (final id order), summed over each cluster's entries in list order
    std::vector<double> birth(ncl), st(ncl, 0.0);
    std::vector<int64_t> par(ncl), k0(ncl, -1), k1(ncl, -1);
    for (int64_t c = 0; c < ncl; ++c) {
        const int64_t i = fid[c] - n;
        birth[i] = T.birth[c];
        par[i] = T.parent[c] < 0 ? -1 : fid[T.parent[c]] - n;
    }
    for (int64_t i = 1; i < ncl; ++i) (k0[par[i]] < 0 ? k0[par[i]] : k1[par[i]]) = i; // ascending: k0 < k1
    for (int64_t j = 0; j < ne; ++j) {
        const Entry &r = T.raw[at[j]];
        const int64_t i = (int64_t)(key[j] >> cb);
        if (r.lambda != birth[i]) st[i] += (double)r.size * (r.lambda - birth[i]);
    }

    // excess of mass, children first; the root is never selected
    std::vector<double> best(ncl);
    std::vector<char> keep(ncl, 0);
    for (int64_t i = ncl - 1; i >= 0; --i) {
        double sub = 0.0;
        if (k0[i] >= 0) {
            sub += best[k0[i]];
            sub += best[k1[i]];
        }
        if (i > 0 && st[i] >= sub) {
            keep[i] = 1;
            best[i] = st[i];
        } else {
            best[i] = sub;
        }
    }
    // selection (a kept cluster with no kept ancestor) and cluster labels, parents first
    std::vector<char> covered(ncl, 0);
    std::vector<int32_t> clab(ncl, -1);
    int32_t nsel = 0;
    for (int64_t i = 0; i < ncl; ++i) {
        const int64_t p = par[i];
        covered[i] = p >= 0 && (covered[p] || keep[p]);
        if (keep[i] && !covered[i])
            clab[i] = nsel++;
        else
            clab[i] = p >= 0 ? clab[p] : -1;
    }
    for (int64_t j = 0; j < ne; ++j) {
        const int64_t child = (int64_t)(key[j] & cmask);
        if (child < n) out_labels[child] = clab[key[j] >> cb];
    }

    if (want_tree)
        for (int64_t j = 0; j < ne; ++j) {
            const Entry &r = T.raw[at[j]];
            ct_parent[j] = n + (int64_t)(key[j] >> cb);
            ct_child[j] = (int64_t)(key[j] & cmask);
            ct_lambda[j] = r.lambda;
            ct_size[j] = r.size;
        }
    if (out_stability) std::copy(st.begin(), st.end(), out_stability);
    if (info) *info = ekh_hdbscan_info{ne, (int32_t)ncl, nsel};
    return EKH_OK;
}
