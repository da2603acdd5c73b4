/*
 * ekh.h -- C ABI of libekh.so: exact k-nearest neighbours, HDBSCAN core
 * distances and the Boruvka minimum spanning tree of the mutual-reachability
 * graph, on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; section names as printed there):
 *  - "Kilosort4 clustering and matching", section "k-nearest neighbours are a
 *    matrix product": squared distances as |x|^2 + |y|^2 - 2 x.y, one dense
 *    product plus two norm vectors, a per-row keep-the-k-smallest step,
 *    feature-major storage [d, n] used without a copy, rows processed in chunks
 *    so the per-launch scratch stays bounded (MAX_CHUNK_DOTS).
 *  - "HDBSCAN", section "The algorithm on the device": core distance = distance
 *    to the min_samples-th nearest neighbour with the point itself included;
 *    MST of max(core_a, core_b, |a - b|) by Boruvka rounds; ordering edges by
 *    (weight, lower index, higher index) leaves exactly one minimum tree.
 *  - same page, section "The hang": the nearest list is a fixed,
 *    compile-time-unrolled compare-and-swap sequence, no flag-terminated loop;
 *    every kernel loop is bounded by a counter or a constant.
 *  - same page, section "Exact shortcuts": neighbour-edge candidates (a list of
 *    min_samples + 1 neighbours proves completeness) and the per-component
 *    upper bound that lets clips skip the all-points scan.
 *
 * Conventions shared by every entry point
 *  - Point sets are feature-major: point i of X has feature f at
 *    X[f * ldx + i] (any n, m, d and ld, odd values included), with
 *    n <= ldx < 2^48 and d <= EKH_MAX_DIM = 256, the widest form the tile
 *    kernels hold in registers (a limit the pages do not set; their sets
 *    have 60 to 200 features).  The calls read the database through a
 *    point-major copy in the workspace, so the leading dimension does not
 *    enter any tile address.
 *    X, Y, outputs and the workspace are DEVICE pointers owned by the caller;
 *    the library never allocates or frees caller memory.
 *  - State kept between calls (a reading; the pages are silent on it): the
 *    optional kernel timer below, the static scratch of ekh_knn_noalloc, and
 *    one extra stream per device (non-blocking, default priority, created on
 *    the first chunked ekh_knn call and kept to the end of the process).  On
 *    it a second row chunk runs beside the caller's stream, forked from and
 *    joined back to the caller's stream with events, so to the caller all
 *    work is ordered on `stream`.  Two chunks in flight took the wide section
 *    (200,000 x 20,000, 63 chunks) from 24.9 to 21.3 ms; taking the stream
 *    from the caller instead would add an argument for that one case.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    ekh_knn and ekh_core_distances do not synchronise the host.
 *    ekh_mst_boruvka blocks: it reads its counters back once per round.
 *  - Squared distances are float32, D2 = max(0, (|x|^2 + |y|^2) - 2 x.y), with
 *    the product on MFMA and the norms computed by the same MFMA contraction
 *    (same feature order), so that D2(a, b) is bitwise symmetric, identical in
 *    every entry point, and exactly 0 for bitwise-identical points.
 *    Distances are the correctly rounded square root of D2.
 *  - Neighbour rows are ascending under (D2, index): equal distances keep the
 *    lower index first.
 *  - Return value: EKH_OK (0) or a negative code; ekh_last_error() then holds a
 *    message (thread-local).  Argument errors are detected before any GPU work.
 *    Inputs must be finite.
 */
#ifndef EKH_H
#define EKH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EKH_OK 0
#define EKH_EINVAL (-1)     /* bad argument: null pointer, size out of range, ld < n, ... */
#define EKH_EWORKSPACE (-2) /* ws_bytes smaller than the matching *_workspace_bytes() */
#define EKH_EHIP (-3)       /* a HIP runtime call failed; message names it */
#define EKH_EINTERNAL (-4)  /* Boruvka round cap exceeded or a component found no edge */

#define EKH_MAX_K 32      /* largest k (and min_samples + 1) */
#define EKH_MAX_DIM 256   /* largest d */
#define EKH_MAX_ROUNDS 64 /* size of the per-round statistics arrays */

/* Library version, major * 10000 + minor * 100 + patch. */
int ekh_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char *ekh_last_error(void);

/* ------------------------------------------------------------------ kNN */

/*
 * Workspace bytes ekh_knn needs for these sizes (max_chunk_dots as in ekh_knn).
 */
size_t ekh_knn_workspace_bytes(int64_t n, int64_t m, int32_t d, int32_t k, int64_t max_chunk_dots);

/*
 * For each of the n points of X, the k nearest of the m points of Y
 * ("k-nearest neighbours are a matrix product").
 *
 *  X [d, n] (ld ldx), Y [d, m] (ld ldy): float32 device arrays.  If Y == X
 *      (same pointer, ld and size) the set is its own database and the pair
 *      (i, i) has D2 = 0 exactly; otherwise no pair is special.
 *  k: 1 <= k <= min(m, EKH_MAX_K).  d: 1 <= d <= EKH_MAX_DIM.
 *  out_idx [n, k] int32 (row-major): indices into Y.  out_dist [n, k]
 *      float32.  Either may be NULL.  The k neighbours are the k smallest under
 *      (D2, index) with D2 in the GEMM form above; their reported distance is
 *      sqrt_rn of D2 recomputed by direct differences, sum_f (x_f - y_f)^2 with
 *      fmaf in feature order (free of the GEMM form's cancellation error), and
 *      each row is ascending under (that D2, index).
 *  max_chunk_dots: if > 0, the rows go in chunks of at most
 *      max_chunk_dots / m rows (at least one row tile), each chunk a separate
 *      launch sequence whose scratch is sized for that chunk (MAX_CHUNK_DOTS on
 *      the page); 0 = one chunk.  Results do not depend on it.
 *  ws, ws_bytes: device scratch of at least ekh_knn_workspace_bytes() (norms,
 *      split lists, the list indices when out_idx is NULL, and a point-major
 *      copy of Y [m, 16 ceil(d / 16)] that the tiles stream and the reported
 *      distances gather from).
 */
int ekh_knn(const float *X, int64_t ldx, int64_t n, const float *Y, int64_t ldy, int64_t m, int32_t d, int32_t k,
            int32_t *out_idx, float *out_dist, int64_t max_chunk_dots, void *ws, size_t ws_bytes, void *stream);

/*
 * Launch layout the kNN tile kernel takes for these sizes (host only, no GPU
 * call; ekh_knn, ekh_core_distances and ekh_mst_boruvka plan through the same
 * function, the last two with m = n and max_chunk_dots = 0).  The query rows go
 * in chunks; each chunk is one launch whose query tiles (64 or 128 rows) either
 * all read the database in the same number of splits, or (when a last round of
 * resident workgroups would be ragged) the first body tiles read the whole
 * database and only the rest are split.  Up to 2 chunks are in flight at once,
 * each on its own stream (the caller's and streams the library creates once per
 * device, joined back to the caller's stream with events) and scratch, and each
 * sized to its share of the resident workgroups.  Split lists are merged by one
 * more launch; results never depend on the layout.
 *  out[0] rows per chunk, out[1] query rows per tile, out[2] body tiles of the
 *  first chunk, out[3] database splits of its other tiles, out[4] resident
 *  workgroups per chunk in flight, out[5] body tiles of the last chunk,
 *  out[6] its splits, out[7] chunks in flight.
 * Returns EKH_OK, or EKH_EINVAL for sizes ekh_knn rejects or a NULL out.
 */
int ekh_knn_plan(int64_t n, int64_t m, int32_t d, int32_t k, int64_t max_chunk_dots, int64_t out[8]);

/*
 * ekh_knn without a workspace or any allocation, for callers that cannot call
 * hipMalloc (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments and results as ekh_knn, bit for bit,
 * except ws and ws_bytes: its scratch is a static device array of
 * EKH_NOALLOC_SCRATCH_BYTES held by every GPU the library runs on until the
 * process ends, and every chunk runs on `stream` (no second stream, no event).
 * Sizes whose scratch (ekh_knn_noalloc_bytes) exceeds the array return
 * EKH_EWORKSPACE with a message.  All calls on one GPU share that GPU's array
 * (it keeps the last call's contents; nothing in it needs clearing): calls
 * that overlap on one GPU race and must be ordered by the caller, e.g. on one
 * stream.  Other errors as ekh_knn.
 */
#define EKH_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t ekh_knn_noalloc_bytes(int64_t n, int64_t m, int32_t d, int32_t k, int64_t max_chunk_dots);
int ekh_knn_noalloc(const float *X, int64_t ldx, int64_t n, const float *Y, int64_t ldy, int64_t m, int32_t d,
                    int32_t k, int32_t *out_idx, float *out_dist, int64_t max_chunk_dots, void *stream);

/* ------------------------------------------------------------------ core distances */

size_t ekh_core_workspace_bytes(int64_t n, int32_t d, int32_t min_samples);

/*
 * Core distance of every point of X: the distance to its min_samples-th nearest
 * point, the point itself counted ("HDBSCAN", "The algorithm on the device").
 * Computed as the self-kNN of X with K = min_samples + 1 entries (the extra
 * entry serves the neighbour-edge shortcut of ekh_mst_boruvka).
 *
 *  min_samples: 1 <= min_samples <= n - 1 and min_samples + 1 <= EKH_MAX_K.
 *  out_core [n] float32 (required): the min_samples-th smallest (from 1) of
 *      the row's K = min_samples + 1 list entries' distances recomputed by direct
 *      differences, sqrt_rn(sum_f (x_f - y_f)^2) with fmaf in feature order.
 *      The GEMM form's cancellation error (about 1e-5 relative for points whose
 *      norm is large against their neighbour distance) does not reach it; the
 *      list's extra entry keeps the rank-min_samples point in the list even
 *      when that error reorders ranks min_samples and min_samples + 1.
 *  out_nbr_idx [n, min_samples + 1] int32, out_nbr_d2 [n, min_samples + 1]
 *      float32 (both NULL or both set): the self-kNN rows, ascending under
 *      (D2, index), self included with D2 = 0; D2 here is the GEMM form, the
 *      value ekh_mst_boruvka's scan computes for the same pair bit for bit.
 *  ws: at least ekh_core_workspace_bytes() (norms, split lists, a point-major
 *      copy of X [n, 16 ceil(d / 16)] that the tiles stream and the direct
 *      differences gather from, and the list indices).
 *
 * From 16,384 points on at d <= 64 the self-kNN computes every pair once
 * (D2 is bitwise symmetric): a bound pass finds each point's (min_samples + 1)-th
 * nearest among every 16th point, a bound on its final one; the symmetric
 * pass runs each query block over its own and the later blocks' points, a
 * pair feeding the query's list and, within the later point's bound, that
 * point's candidate buffer (512 entries per point in the workspace, 4 KB);
 * the lists are then merged, and a query block with an overflowed buffer is
 * recomputed from both sides.  The lists are the same bit for bit as with
 * every pair computed from both sides, which the environment variable
 * EKH_CORE_DENSE (set and not "0") selects instead; the workspace query and
 * the call must see the same setting.  (A reading: the pages compute every
 * pair of the core-distance kernel; symmetry changes no result.)
 */
int ekh_core_distances(const float *X, int64_t ldx, int64_t n, int32_t d, int32_t min_samples, float *out_core,
                       int32_t *out_nbr_idx, float *out_nbr_d2, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ Boruvka MST */

/* flags for ekh_mst_boruvka: switch the exact shortcuts off (results do not change) */
#define EKH_MST_NO_NEIGHBOUR_EDGES 1u
#define EKH_MST_NO_COMPONENT_BOUND 2u
/* scan the largest component's active points against all points, not only
   against the points outside it (used when it holds at least n / 2 points) */
#define EKH_MST_FULL_SCANS 4u

typedef struct {
    int32_t rounds;                          /* Boruvka rounds run */
    int32_t n_components[EKH_MAX_ROUNDS];    /* components after each round */
    int64_t resolved[EKH_MAX_ROUNDS];        /* points whose cheapest edge came from their list */
    int64_t skipped[EKH_MAX_ROUNDS];         /* points skipped by the component bound */
    int64_t scanned[EKH_MAX_ROUNDS];         /* points scanned */
    int64_t edges_added[EKH_MAX_ROUNDS];
    double round_ms[EKH_MAX_ROUNDS];         /* host wall time of each round */
    int64_t scanned_giant[EKH_MAX_ROUNDS];   /* of the scanned, points of a component holding >= n / 2
                                                points, scanned only against the points outside it */
} ekh_mst_stats;

size_t ekh_mst_workspace_bytes(int64_t n, int32_t d, int32_t min_samples, int with_neighbours);

/*
 * Minimum spanning tree of the complete graph on the n points of X with weight
 * W(a, b) = max(core_a, core_b, sqrt_rn(D2(a, b))), ties broken by (W, lower
 * index, higher index), by Boruvka rounds with the exact shortcuts of
 * "Exact shortcuts" ("HDBSCAN" page).
 *
 *  D2 is the GEMM form, the value ekh_core_distances' lists hold for the same
 *  pair bit for bit, so the list shortcuts and the scan weigh every edge alike.
 *
 *  core [n] float32: core distances as given (normally ekh_core_distances).
 *  nbr_idx, nbr_d2 [n, min_samples + 1]: the self-kNN rows ekh_core_distances
 *      returns; if both NULL they are recomputed inside (with_neighbours = 0
 *      in the workspace query).  The shortcuts are exact for any core array:
 *      a list holds every point closer than its last entry, so a point whose
 *      lightest edge into its list is lighter than that entry's distance needs
 *      no scan, and a point whose core distance or last-entry distance exceeds
 *      its component's lightest known edge cannot supply a lighter one.
 *  flags: EKH_MST_NO_* and EKH_MST_FULL_SCANS switches (none changes the tree;
 *      EKH_MST_NO_NEIGHBOUR_EDGES stops every use of the lists' completeness).
 *      From the second round on, when one component holds at least n / 2
 *      points, its active points are scanned only against a gathered copy of
 *      the points outside it (the workspace holds d * (n / 2 + 1) floats for
 *      that copy).
 *  out_lo, out_hi [n - 1] int32, out_w [n - 1] float32: the edges, lo < hi,
 *      sorted by (w, lo, hi).  The tree is the minimum one under the W above;
 *      each reported w is max(core_lo, core_hi, D) with D recomputed by direct
 *      differences (sqrt_rn of sum_f (x_lo,f - x_hi,f)^2, fmaf in feature
 *      order), free of the GEMM form's cancellation error.  n = 1 gives no
 *      edges.
 *  stats: optional host struct filled per round.
 *  Blocks the host once per round (one read-back of the round's counters);
 *  the scans find the number of points to scan on the device.
 *  ws: at least ekh_mst_workspace_bytes() (round state, a point-major copy
 *      of X [n, 16 ceil(d / 16)] that the scans stream and the reported weights
 *      gather from, the gathered complement of the largest component, sort
 *      buffers, and the lists when they are recomputed).
 *  Requires 1 <= min_samples < n for n >= 2.  At most ceil(log2 n) rounds;
 *  more returns EKH_EINTERNAL.
 */
int ekh_mst_boruvka(const float *X, int64_t ldx, int64_t n, int32_t d, const float *core, int32_t min_samples,
                    const int32_t *nbr_idx, const float *nbr_d2, uint32_t flags, int32_t *out_lo, int32_t *out_hi,
                    float *out_w, ekh_mst_stats *stats, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ kernel timer (measurement) */

/*
 * Bipartite kNN-graph assignment (device).  Source: "Kilosort4 clustering and
 * matching", section "Assignment in parallel: why the graph is bipartite".
 * Left nodes are n spikes, right nodes m subset points; nbr [n, k] (row-major
 * int32, each row a spike's neighbours among the subset, e.g. the out_idx of
 * ekh_knn(X = spikes, Y = subset, k)) gives the edges.  Rounds alternate a left
 * step (every spike takes the best label among its neighbours' right labels)
 * and a right step (integer atomic counts[r, label] over the edges, then every
 * right node takes the best label among its neighbours' left labels).  Score of
 * label c for node v: n_vc - gamma k_v K_c / (2 m_e), float64 in that order,
 * with n_vc the neighbours of v labelled c, k_v the degree of v (k for a spike,
 * the number of spikes listing r for a right node), m_e = n k, and K_c the total
 * degree of the OTHER side's nodes labelled c.  Readings where the page is
 * silent: candidates are the labels present among the node's neighbours; ties
 * keep the current label if it is among the best, else take the smallest;
 * spikes start unlabelled; right nodes start from init_right; the loop stops
 * after a left step that moves no spike, or after max_rounds rounds (the page:
 * a 200-round cap); a right node that no spike lists keeps its label.
 *
 * init_right [m] int32 labels in [0, n_clusters); out_left [n], out_right [m]
 * int32 (device, caller-owned); out_rounds (HOST, nullable) receives the rounds
 * run.  Workspace: ekh_bipartite_workspace_bytes(m, n_clusters) bytes
 * (4 (m + 2 C + m C) plus alignment).  Blocks: one 4-byte read-back per round.
 * Errors: EKH_EINVAL for a NULL array, n, m < 1, k outside [1, 32],
 * n_clusters < 1, n k or m n_clusters >= 2^31, gamma negative or not finite,
 * max_rounds < 1, or (checked on the device before any step) a neighbour index
 * outside [0, m) or a starting label outside [0, n_clusters); EKH_EWORKSPACE;
 * EKH_EHIP.
 */
size_t ekh_bipartite_workspace_bytes(int64_t m, int32_t n_clusters);
int ekh_bipartite_assign(const int32_t *nbr, int64_t n, int32_t k, int64_t m, int32_t n_clusters,
                         const int32_t *init_right, double gamma, int32_t max_rounds, int32_t *out_left,
                         int32_t *out_right, int32_t *out_rounds, void *ws, size_t ws_bytes, void *stream);

/*
 * Edge counts between clusters (device).  Source: "Kilosort4 clustering and
 * matching", section "Merges and splits": the merging tree is built from the
 * cluster-to-cluster edge counts alone, which one pass of atomic adds fills on
 * the device and the host copies back once.  out_counts [C, C] u32 (device, row-major, written
 * whole): out_counts[a * C + b] = number of edges (spike i, subset point r) of
 * nbr [n, k] with left[i] = a and right[r] = b.  ws: at least 16 bytes of device
 * memory.  Blocks: three range counters are read back before any count is
 * added.  Errors: EKH_EINVAL for a NULL array, sizes out of range
 * (n_clusters > 46340, n k >= 2^31), neighbour indices outside [0, m) or labels
 * outside [0, n_clusters); EKH_EWORKSPACE; EKH_EHIP.
 */
int ekh_cluster_edge_counts(const int32_t *nbr, int64_t n, int32_t k, int64_t m, const int32_t *left,
                            const int32_t *right, int32_t n_clusters, uint32_t *out_counts, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Merging tree of the clusters, on the HOST (same section: building it is host
 * work).  The page does not give the rule; this is greedy modularity
 * agglomeration in the terms of the assignment above:
 *  - the cluster graph is undirected, W[a, b] = counts[a, b] + counts[b, a];
 *    M = total edges; K[a] = row sum + column sum of a (every edge adds one end
 *    to its left label and one to its right label);
 *  - each step merges the live pair a < b with the largest
 *    dQ = W[a, b] / M - gamma K[a] K[b] / (2 M^2) (float64 in that order; 0
 *    when M = 0); ties go to the smallest (a, b); the merged cluster keeps the
 *    id a (W[a, .] += W[b, .], W[., a] += W[., b], K[a] += K[b]);
 *  - all C - 1 merges are made, so the result is a full binary tree.
 * counts [C, C] u32 HOST (e.g. ekh_cluster_edge_counts copied back);
 * out_a, out_b [C - 1] int32 and out_gain [C - 1] float64 HOST, in merge order.
 * Errors: EKH_EINVAL for a NULL array, n_clusters outside [1, 46340], gamma
 * negative or not finite.  No GPU work; thread-safe.
 */
int ekh_merge_tree(const uint32_t *counts, int32_t n_clusters, double gamma, int32_t *out_a, int32_t *out_b,
                   double *out_gain);

/*
 * Greedy k-means++ seeding of a section.  Source: "Kilosort4 clustering and
 * matching", section "The measurement that changed the design: serial chains
 * inside a thread": every seed after the first is picked from 2 + ln k
 * candidates sampled with squared-distance weights, keeping the one that
 * leaves the lowest potential; the random numbers come from the host in one
 * upload, and sampling, scoring and picking all run on the device without
 * waiting on the host.  The page leaves
 * the arithmetic open; the conventions here make every decision exact:
 *  - L = 2 + floor(ln k) candidates per seed after the first (7 at k = 200);
 *  - squared distances are float32, summed over features in order from 0,
 *    every subtraction, product and sum rounded (nothing fused);
 *  - with D1 the squared distances to the first seed and 2^(e-1) <= max D1
 *    < 2^e, S = 40 - e (0 when max D1 = 0); a squared distance D has the
 *    integer weight floor(D 2^S), and w(x) is point x's weight to its
 *    nearest seed so far; all sums are exact 64-bit integers;
 *  - only the low 53 bits of each uniform are used (u in [0, 2^53)), in order:
 *    uniforms[0] gives the first seed, point floor(u n / 2^53); seed s >= 1
 *    draws its candidates j = 0..L-1 from uniforms[1 + (s - 1) L + j];
 *  - a candidate is the first point whose inclusive prefix sum of w exceeds
 *    floor(u T / 2^53), T = sum of w (point 0 when T = 0);
 *  - a candidate's potential is sum_x min(w(x), floor(D(x, cand) 2^S)); the
 *    smallest wins, ties going to the candidate drawn first.
 * X [d, n] float32 device, feature-major with leading dimension ldx >= n;
 * uniforms [n_uniforms] device, n_uniforms >= 1 + (k - 1) L; out_seeds [k]
 * int32 device (point indices in seed order; a seed repeats only when every
 * weight is 0, e.g. fewer than k distinct points); out_potential (device, one
 * int64, nullable): the final sum of w.
 * Two paths with identical results: sections with n <= 4096,
 * n <= 4 (1 + (k - 1) L) and L <= 7 (k <= 403) compute the n x n matrix of squared
 * distances once (n^2 4 bytes of workspace) and seed in one persistent
 * block (2 launches in all); otherwise, or with flags
 * EKH_KMEANSPP_PER_SEED_LAUNCHES, two launches per seed (about 24 n bytes of
 * workspace).  Workspace: ekh_kmeanspp_workspace_bytes(n, k, flags) bytes of
 * device memory (0 for arguments out of range).  Enqueued on `stream`, no
 * host sync.  Inputs must be finite (not checked).
 * Errors: EKH_EINVAL for a NULL array, n outside [1, 2^22], d outside
 * [1, 8192], k outside [1, 2^20], ldx outside [n, 2^25), unknown flags or
 * too few uniforms; EKH_EWORKSPACE; EKH_EHIP.
 */
#define EKH_KMEANSPP_PER_SEED_LAUNCHES 1u
size_t ekh_kmeanspp_workspace_bytes(int64_t n, int32_t k, uint32_t flags);
int ekh_kmeanspp(const float *X, int64_t ldx, int64_t n, int32_t d, int32_t k, const uint64_t *uniforms,
                 int64_t n_uniforms, uint32_t flags, int32_t *out_seeds, int64_t *out_potential, void *ws,
                 size_t ws_bytes, void *stream);

/*
 * HDBSCAN tail, on the HOST: spanning tree -> single-linkage hierarchy ->
 * condensed tree -> excess-of-mass selection -> cluster labels.
 * Source: "HDBSCAN", section "The algorithm on the device", last item (the
 * page does the single-linkage hierarchy, its condensing and the
 * excess-of-mass choice on the CPU, in time linear in n) with the edge order
 * of the same section; the steps
 * are the standard HDBSCAN* definitions, with these conventions:
 *  - the n - 1 edges are merged in ascending (w, lo, hi) order, one union each
 *    (equal weights thus merge in index order, like the tree's own tie rule);
 *  - lambda = 1 / w (float64; +inf for w = 0);
 *  - walking the hierarchy down inside a cluster, a merge's child with at least
 *    min_cluster_size points is large: both large -> two clusters are born at
 *    that lambda; one large -> the other child's points leave at lambda; none
 *    -> all points leave at lambda;
 *  - clusters are numbered n (root), n + 1, ... breadth-first, the two children
 *    of a split by ascending smallest point index;
 *  - stability(c) = sum of size * (lambda - birth(c)) over c's condensed-tree
 *    entries in ascending (parent, child) order, a term being 0 when lambda ==
 *    birth(c);
 *  - excess of mass, children first: a non-root cluster is kept when its
 *    stability is >= the sum of its two children's best values (ties keep the
 *    parent); the root is never selected; the selection is the kept clusters
 *    with no kept ancestor, labelled 0, 1, ... in ascending id;
 *  - a point's label is that of the selected cluster above it, else -1 (noise).
 *
 * lo, hi [n-1] int32 (lo < hi), w [n-1] float32: a spanning tree, e.g. the
 *   output of ekh_mst_boruvka copied to the host (any edge order is accepted;
 *   sorted input is used as is).  Host pointers, caller-owned, read only.
 * out_labels [n] int32: host, written.
 * ct_parent, ct_child, ct_size [2n] int64 and ct_lambda [2n] float64: the
 *   condensed tree (children: point indices < n or cluster ids >= n), rows in
 *   ascending (parent, child) order; all four NULL to skip.
 * out_stability [n] float64 (nullable): stability of cluster n + i at [i].
 * info (nullable): entries written, clusters in the condensed tree (root
 *   included), clusters selected.
 * Errors: EKH_EINVAL for n < 1, min_cluster_size < 2, a NULL array, lo >= hi
 *   or out of range, a weight that is negative, NaN or infinite, or edges that
 *   do not form a spanning tree.  No GPU work; thread-safe.
 */
typedef struct {
    int64_t n_entries;  /* rows of the condensed tree */
    int32_t n_clusters; /* clusters in the condensed tree, root included */
    int32_t n_selected; /* clusters selected (labels 0 .. n_selected - 1) */
} ekh_hdbscan_info;

int ekh_hdbscan_tail(const int32_t *lo, const int32_t *hi, const float *w, int64_t n, int32_t min_cluster_size,
                     int32_t *out_labels, int64_t *ct_parent, int64_t *ct_child, double *ct_lambda, int64_t *ct_size,
                     double *out_stability, ekh_hdbscan_info *info);

/*
 * Optional per-kernel timing with HIP events recorded on the launch stream
 * around every launch of the two dense kernels, for roofline figures.
 * kernel id: 0 = the kNN tile kernel (with the bound pass of ekh_core_distances'
 * symmetric self-kNN), 1 = the Boruvka scan tile kernel, 2 = the symmetric
 * self-kNN kernel (its flop: 2 d per pair it computes, each once).
 * ekh_timer_enable(1) clears and starts recording; ekh_timer_read() waits for
 * the recorded events and returns the launch count, summed milliseconds and
 * summed algorithmic flop (2 d per distance pair actually evaluated, padding
 * excluded).  Returns EKH_EINVAL for an unknown id.
 */
int ekh_timer_enable(int on);
int ekh_timer_read(int kernel_id, int64_t *launches, double *total_ms, double *algo_flop);

#ifdef __cplusplus
}
#endif

#endif /* EKH_H */
