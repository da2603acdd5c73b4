// Instantiation of the kNN tile and merge kernels for one list length K (the
// tile kernel once per k-step count QM).  Compiled once per K with
// -DEKH_KNN_K=<K> (2, 4, 8, 10, 11, 16, 32), so the instantiations build in
// parallel.
#include "tile_common.h"

#ifndef EKH_KNN_K
#error "compile with -DEKH_KNN_K=<list length>"
#endif

namespace ekh {

namespace {
template <int K, int QM> hipError_t knn_tile_launch(const KnnArgs &a, hipStream_t s) {
    constexpr int CB = knn_col_blocks(K, QM);
    constexpr int QT = kWaves * 16 * CB;
    const int64_t tail_q = (a.nq - a.body_q * QT + QT - 1) / QT;
    const int64_t groups = a.body_q + tail_q * a.splits;
    if (a.body_q < 0 || tail_q < 0 || a.splits < 1 || groups > 0x7fffffff || a.dp != tile_dim(a.d) ||
        pick_qm(a.d) != QM)
        return hipErrorInvalidValue;
    // the bound pass (d <= 64) keeps values only
    if constexpr (QM <= 16)
        if (a.out_mode == kOutBound) {
            hipLaunchKernelGGL((knn_tile_kernel<K, QM, true>), dim3((unsigned)groups), dim3(kThreads), 0, s, a);
            return hipGetLastError();
        }
    hipLaunchKernelGGL((knn_tile_kernel<K, QM>), dim3((unsigned)groups), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}
} // namespace

template <> hipError_t launch_knn_tile_k<EKH_KNN_K>(int QM, const KnnArgs &a, hipStream_t s) {
    switch (QM) {
#define EKH_KNN_TILE_CASE(q)                                                                                           \
    case q: return knn_tile_launch<EKH_KNN_K, q>(a, s);
        EKH_FOR_EACH_QM(EKH_KNN_TILE_CASE)
#undef EKH_KNN_TILE_CASE
    default: return hipErrorInvalidValue;
    }
}

template <> hipError_t launch_knn_sym_k<EKH_KNN_K>(int QM, const KnnArgs &a, hipStream_t s) {
    // the symmetric pass runs at d <= 64 only (the planner's choice); one
    // instantiation per list length
    const int64_t QT = sym_query_tile(EKH_KNN_K, QM);
    const int64_t groups = (a.nq + QT - 1) / QT * a.splits;
    if (a.splits < 1 || groups > 0x7fffffff || a.dp != tile_dim(a.d) || pick_qm(a.d) != QM || a.m != a.nq ||
        a.colcap < 1 || !a.tau || !a.theta || !a.colbuf || !a.colcnt || !a.part)
        return hipErrorInvalidValue;
    switch (QM) {
#define EKH_KNN_SYM_CASE(q)                                                                                            \
    case q: hipLaunchKernelGGL((knn_sym_kernel<EKH_KNN_K, q>), dim3((unsigned)groups), dim3(kThreads), 0, s, a); break;
        EKH_KNN_SYM_CASE(2) EKH_KNN_SYM_CASE(4) EKH_KNN_SYM_CASE(6) EKH_KNN_SYM_CASE(8) EKH_KNN_SYM_CASE(10)
        EKH_KNN_SYM_CASE(12) EKH_KNN_SYM_CASE(14) EKH_KNN_SYM_CASE(16)
#undef EKH_KNN_SYM_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <> hipError_t launch_sym_merge_k<EKH_KNN_K>(const KnnArgs &a, hipStream_t s) {
    if (a.nq <= 0 || !a.gate_w || a.gate_rows < 1) return hipErrorInvalidValue;
    const int bs = 256;
    const int64_t threads = a.nq * kMergeLanes;
    hipLaunchKernelGGL(sym_merge_kernel<EKH_KNN_K>, dim3((unsigned)((threads + bs - 1) / bs)), dim3(bs), 0, s, a);
    return hipGetLastError();
}

template <> hipError_t launch_knn_rescore_k<EKH_KNN_K>(const KnnArgs &a, hipStream_t s) {
    constexpr int rows = DirectRows<EKH_KNN_K>::kRowsPerBlock;
    if (a.dp > kDirectMaxDim || a.k_out > EKH_KNN_K) return hipErrorInvalidValue;
    hipLaunchKernelGGL(knn_rescore_kernel<EKH_KNN_K>, dim3((unsigned)((a.nq + rows - 1) / rows)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <> hipError_t launch_knn_core_k<EKH_KNN_K>(const KnnArgs &a, hipStream_t s) {
    constexpr int rows = DirectRows<EKH_KNN_K>::kRowsPerBlock;
    if (a.dp > kDirectMaxDim || a.k_out > EKH_KNN_K || a.min_samples < 1 || a.min_samples > a.k_out)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(knn_core_kernel<EKH_KNN_K>, dim3((unsigned)((a.nq + rows - 1) / rows)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <> hipError_t launch_knn_merge_k<EKH_KNN_K>(const KnnArgs &a, hipStream_t s) {
    const int bs = 256;
    const int64_t threads = a.nq * kMergeLanes;
    hipLaunchKernelGGL(knn_merge_kernel<EKH_KNN_K>, dim3((unsigned)((threads + bs - 1) / bs)), dim3(bs), 0, s, a);
    return hipGetLastError();
}

} // namespace ekh
