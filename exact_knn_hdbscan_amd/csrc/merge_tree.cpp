// Host merging tree of libekh (ekh_merge_tree).
//
// Kilosort4 clustering page, section "Merges and splits": the tree is built on
// the host from nothing but the cluster-to-cluster edge counts (a matrix of at
// most 200 x 200, copied back from the device once).  The merging rule is greedy modularity
// agglomeration on the undirected cluster graph, with the conventions stated
// in include/ekh.h.  O(C^3) for C clusters (8e6 steps at C = 200).  Built with
// -ffp-contract=off so that every gain rounds as written.
#include "ekh.h"
#include "host_error.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
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

// dQ = W / M - gamma K_a K_b / (2 M^2), in this order; 0 when there are no edges
inline double merge_gain(int64_t w_ab, int64_t k_a, int64_t k_b, int64_t m_total, double gamma) {
    if (m_total == 0) return 0.0;
    const double m = (double)m_total;
    return (double)w_ab / m - gamma * (double)k_a * (double)k_b / (2.0 * m * m);
}

} // namespace

extern "C" int ekh_merge_tree(const uint32_t *counts, int32_t n_clusters, double gamma, int32_t *out_a,
                              int32_t *out_b, double *out_gain) {
    if (!counts || (n_clusters > 1 && (!out_a || !out_b || !out_gain))) return fail(EKH_EINVAL, "NULL array");
    if (n_clusters < 1 || n_clusters > 46340) return fail(EKH_EINVAL, "n_clusters = %d out of range", n_clusters);
    if (!(gamma >= 0.0) || std::isinf(gamma)) return fail(EKH_EINVAL, "gamma must be finite and >= 0");
    const int64_t C = n_clusters;
    std::vector<int64_t> W((size_t)(C * C)), K((size_t)C, 0);
    int64_t M = 0;
    for (int64_t a = 0; a < C; ++a)
        for (int64_t b = 0; b < C; ++b) {
            const int64_t c = counts[a * C + b];
            M += c;
            W[a * C + b] += c; // W = counts + counts^T
            W[b * C + a] += c;
            K[a] += c;         // one end on the left label ...
            K[b] += c;         // ... and one on the right label
        }
    std::vector<char> alive((size_t)C, 1);
    for (int64_t step = 0; step + 1 < C; ++step) {
        int64_t ba = -1, bb = -1;
        double bg = 0.0;
        for (int64_t a = 0; a < C; ++a) {
            if (!alive[a]) continue;
            for (int64_t b = a + 1; b < C; ++b) {
                if (!alive[b]) continue;
                const double g = merge_gain(W[a * C + b], K[a], K[b], M, gamma);
                if (ba < 0 || g > bg) { // lexicographic order: the first best is the smallest pair
                    ba = a;
                    bb = b;
                    bg = g;
                }
            }
        }
        out_a[step] = (int32_t)ba;
        out_b[step] = (int32_t)bb;
        out_gain[step] = bg;
        alive[bb] = 0;
        for (int64_t c = 0; c < C; ++c) W[ba * C + c] += W[bb * C + c];
        for (int64_t c = 0; c < C; ++c) W[c * C + ba] += W[c * C + bb];
        K[ba] += K[bb];
    }
    return EKH_OK;
}
