/*
 * CPU oracle for exact kNN, HDBSCAN core distances and the minimum spanning
 * tree of the mutual-reachability graph.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * Everything is the plain definition, in float64 (inputs are float32 and are
 * widened exactly), with no blocking or reordering beyond a loop over features:
 *
 *   D^2(a, b) = sum_f (a_f - b_f)^2                       (direct differences)
 *   kNN(q)    = the k smallest points under the total order (D^2, index)
 *   core(a)   = sqrt of D^2 to the min_samples-th entry of a's own list, the
 *               point itself counted (HDBSCAN page, "The algorithm on the
 *               device", first item)
 *   W(a, b)   = max(core_a, core_b, D(a, b))  (same page and section, second item)
 *   MST       = the unique spanning tree that is minimal under the edge order
 *               (W, lower index, higher index) (same item: the tie rule that
 *               makes the tree unique)
 *
 * The MST is built twice, by dense Prim and by Kruskal, two independent
 * algorithms whose agreement the tests check.
 *
 * Layout: point sets are feature-major, element (f, i) at X[f * ld + i]
 * (clustering page, "k-nearest neighbours are a matrix product").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* D^2 from point a of A to every point of B, in float64, by direct differences. */
static void sqdist_row(const float *A, int64_t lda, int64_t a, const float *B, int64_t ldb,
                       int64_t m, int d, double *out) {
    for (int64_t j = 0; j < m; ++j) out[j] = 0.0;
    for (int f = 0; f < d; ++f) {
        const double x = (double)A[(int64_t)f * lda + a];
        const float *brow = B + (int64_t)f * ldb;
        for (int64_t j = 0; j < m; ++j) {
            const double t = x - (double)brow[j];
            out[j] += t * t;
        }
    }
}

/* D^2 between two single points. */
double orc_sqdist(const float *A, int64_t lda, int64_t a, const float *B, int64_t ldb, int64_t b, int d) {
    double s = 0.0;
    for (int f = 0; f < d; ++f) {
        const double t = (double)A[(int64_t)f * lda + a] - (double)B[(int64_t)f * ldb + b];
        s += t * t;
    }
    return s;
}

/*
 * k nearest points of Y for each of the n points of X (clustering page, "k-nearest
 * neighbours are a matrix product": every spike linked to its nearest points of
 * the subset).  Rows of out_idx / out_d2 ([n, k] row-major) are ascending under
 * (D^2, index); equal distances go to the lower index.  When Y is X the point
 * itself is part of the candidates (its D^2 is 0).  Requires 1 <= k <= m.
 *
 * Selection: walk j = 0..m-1 in order and keep the k best seen so far, sorted.
 * A later j can only displace an entry with a strictly larger D^2, because on
 * equal D^2 the earlier (lower) index ranks first.
 */
int orc_knn(const float *X, int64_t ldx, int64_t n, const float *Y, int64_t ldy, int64_t m, int d,
            int k, int32_t *out_idx, double *out_d2, int nthreads) {
    if (k < 1 || k > m || d < 1 || n < 0) return -1;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)m);
        double *bd = (double *)malloc(sizeof(double) * (size_t)k);
        int32_t *bi = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        if (!row || !bd || !bi) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < n; ++i) {
                sqdist_row(X, ldx, i, Y, ldy, m, d, row);
                int filled = 0;
                for (int64_t j = 0; j < m; ++j) {
                    const double v = row[j];
                    if (filled == k && !(v < bd[k - 1])) continue;
                    int pos = filled < k ? filled : k - 1;
                    /* shift larger entries one slot to the right */
                    while (pos > 0 && bd[pos - 1] > v) {
                        bd[pos] = bd[pos - 1];
                        bi[pos] = bi[pos - 1];
                        --pos;
                    }
                    bd[pos] = v;
                    bi[pos] = (int32_t)j;
                    if (filled < k) ++filled;
                }
                memcpy(out_d2 + i * k, bd, sizeof(double) * (size_t)k);
                memcpy(out_idx + i * k, bi, sizeof(int32_t) * (size_t)k);
            }
        }
        free(row);
        free(bd);
        free(bi);
    }
    return err;
}

/* Core distance of every point: D to the min_samples-th nearest point, the point
 * itself included (HDBSCAN page, "The algorithm on the device", first item). */
int orc_core_distances(const float *X, int64_t ldx, int64_t n, int d, int min_samples, double *out_core,
                       int nthreads) {
    if (min_samples < 1 || min_samples > n) return -1;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)n * (size_t)min_samples);
    double *d2 = (double *)malloc(sizeof(double) * (size_t)n * (size_t)min_samples);
    if (!idx || !d2) {
        free(idx);
        free(d2);
        return -2;
    }
    int rc = orc_knn(X, ldx, n, X, ldx, n, d, min_samples, idx, d2, nthreads);
    if (rc == 0)
        for (int64_t i = 0; i < n; ++i) out_core[i] = sqrt(d2[i * min_samples + (min_samples - 1)]);
    free(idx);
    free(d2);
    return rc;
}

/* Edge order of the HDBSCAN page ("The algorithm on the device", second item):
 * weight first, then the lower endpoint, then the higher one. */
static int edge_less(double wa, int64_t loa, int64_t hia, double wb, int64_t lob, int64_t hib) {
    if (wa != wb) return wa < wb;
    if (loa != lob) return loa < lob;
    return hia < hib;
}

/*
 * Dense Prim over the complete mutual-reachability graph, O(n^2 d) time, O(n)
 * memory.  key[v] is the smallest edge (W, lo, hi) from the tree to v; each step
 * adds the outside vertex whose key is smallest under the full edge order, so
 * with this strict total order the result is the unique minimum tree.
 * Edges come out in the order Prim adds them: out_lo[e] < out_hi[e].
 */
int orc_prim(const float *X, int64_t ldx, int64_t n, int d, const double *core, int32_t *out_lo,
             int32_t *out_hi, double *out_w, int nthreads) {
    if (n < 1) return -1;
    if (n == 1) return 0;
    set_threads(nthreads);
    double *kw = (double *)malloc(sizeof(double) * (size_t)n);
    int64_t *klo = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    int64_t *khi = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    char *in_tree = (char *)calloc((size_t)n, 1);
    double *d2 = (double *)malloc(sizeof(double) * (size_t)n);
    if (!kw || !klo || !khi || !in_tree || !d2) {
        free(kw); free(klo); free(khi); free(in_tree); free(d2);
        return -2;
    }
    for (int64_t v = 0; v < n; ++v) {
        kw[v] = INFINITY;
        klo[v] = INT64_MAX;
        khi[v] = INT64_MAX;
    }
    int64_t u = 0; /* vertex just added */
    in_tree[0] = 1;
    /* threads per step: one per 2^18 distance terms of the step (the step's
       minimum is taken under a strict total order, so the result does not
       depend on the thread count; small sets then avoid a parallel region's
       start-up cost on each of their n - 1 steps) */
    int nt_step = 1;
#ifdef _OPENMP
    {
        const int64_t want = (n * (int64_t)d) >> 18;
        const int maxt = omp_get_max_threads();
        nt_step = want < 1 ? 1 : (want > maxt ? maxt : (int)want);
    }
#endif
    for (int64_t step = 0; step < n - 1; ++step) {
        int64_t best_v = -1;
        double best_w = INFINITY;
        int64_t best_lo = INT64_MAX, best_hi = INT64_MAX;
#pragma omp parallel num_threads(nt_step)
        {
            int nt = 1, tid = 0;
#ifdef _OPENMP
            nt = omp_get_num_threads();
            tid = omp_get_thread_num();
#endif
            /* this thread's contiguous range of vertices */
            const int64_t v0 = n * tid / nt, v1 = n * (tid + 1) / nt;
            /* D^2(u, v) for v in range, feature by feature (direct differences) */
            for (int64_t v = v0; v < v1; ++v) d2[v] = 0.0;
            for (int f = 0; f < d; ++f) {
                const float *row = X + (int64_t)f * ldx;
                const double xu = (double)row[u];
                for (int64_t v = v0; v < v1; ++v) {
                    const double t = xu - (double)row[v];
                    d2[v] += t * t;
                }
            }
            int64_t tv = -1;
            double tw = INFINITY;
            int64_t tlo = INT64_MAX, thi = INT64_MAX;
            for (int64_t v = v0; v < v1; ++v) {
                if (in_tree[v]) continue;
                double w = sqrt(d2[v]);
                if (core[u] > w) w = core[u];
                if (core[v] > w) w = core[v];
                const int64_t lo = u < v ? u : v, hi = u < v ? v : u;
                if (edge_less(w, lo, hi, kw[v], klo[v], khi[v])) {
                    kw[v] = w;
                    klo[v] = lo;
                    khi[v] = hi;
                }
                if (tv < 0 || edge_less(kw[v], klo[v], khi[v], tw, tlo, thi)) {
                    tv = v;
                    tw = kw[v];
                    tlo = klo[v];
                    thi = khi[v];
                }
            }
#pragma omp critical
            {
                if (tv >= 0 && (best_v < 0 || edge_less(tw, tlo, thi, best_w, best_lo, best_hi))) {
                    best_v = tv;
                    best_w = tw;
                    best_lo = tlo;
                    best_hi = thi;
                }
            }
        }
        out_lo[step] = (int32_t)best_lo;
        out_hi[step] = (int32_t)best_hi;
        out_w[step] = best_w;
        in_tree[best_v] = 1;
        u = best_v;
    }
    free(kw); free(klo); free(khi); free(in_tree); free(d2);
    return 0;
}

/* ---- Kruskal over all n(n-1)/2 edges (small n only) ---- */
typedef struct {
    double w;
    int32_t lo, hi;
} orc_edge;

static int cmp_edge(const void *pa, const void *pb) {
    const orc_edge *a = (const orc_edge *)pa, *b = (const orc_edge *)pb;
    if (edge_less(a->w, a->lo, a->hi, b->w, b->lo, b->hi)) return -1;
    if (edge_less(b->w, b->lo, b->hi, a->w, a->lo, a->hi)) return 1;
    return 0;
}

static int64_t uf_find(int64_t *p, int64_t x) {
    while (p[x] != x) {
        p[x] = p[p[x]];
        x = p[x];
    }
    return x;
}

/* Sort every edge by (W, lo, hi) and keep those that join two trees. */
int orc_kruskal(const float *X, int64_t ldx, int64_t n, int d, const double *core, int32_t *out_lo,
                int32_t *out_hi, double *out_w) {
    if (n < 1 || n > 20000) return -1;
    const int64_t ne = n * (n - 1) / 2;
    orc_edge *e = (orc_edge *)malloc(sizeof(orc_edge) * (size_t)(ne > 0 ? ne : 1));
    int64_t *p = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!e || !p) {
        free(e);
        free(p);
        return -2;
    }
    int64_t t = 0;
    for (int64_t a = 0; a < n; ++a)
        for (int64_t b = a + 1; b < n; ++b) {
            double w = sqrt(orc_sqdist(X, ldx, a, X, ldx, b, d));
            if (core[a] > w) w = core[a];
            if (core[b] > w) w = core[b];
            e[t].w = w;
            e[t].lo = (int32_t)a;
            e[t].hi = (int32_t)b;
            ++t;
        }
    qsort(e, (size_t)ne, sizeof(orc_edge), cmp_edge);
    for (int64_t v = 0; v < n; ++v) p[v] = v;
    int64_t got = 0;
    for (int64_t i = 0; i < ne && got < n - 1; ++i) {
        const int64_t ra = uf_find(p, e[i].lo), rb = uf_find(p, e[i].hi);
        if (ra == rb) continue;
        p[ra] = rb;
        out_lo[got] = e[i].lo;
        out_hi[got] = e[i].hi;
        out_w[got] = e[i].w;
        ++got;
    }
    free(e);
    free(p);
    return got == n - 1 ? 0 : -3;
}

/* Mutual-reachability weight of listed pairs, float64 (for checking trees). */
int orc_pair_weights(const float *X, int64_t ldx, int d, const double *core, int64_t npairs, const int32_t *a,
                     const int32_t *b, double *out_w, double *out_dist, int nthreads) {
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < npairs; ++t) {
        const double dist = sqrt(orc_sqdist(X, ldx, a[t], X, ldx, b[t], d));
        double w = dist;
        if (core[a[t]] > w) w = core[a[t]];
        if (core[b[t]] > w) w = core[b[t]];
        out_w[t] = w;
        if (out_dist) out_dist[t] = dist;
    }
    return 0;
}
