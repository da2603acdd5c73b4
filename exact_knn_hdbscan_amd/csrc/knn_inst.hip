// Instantiation of the kNN tile and merge kernels for one list length K.
// Compiled once per K with -DEKH_KNN_K=<K> (2, 4, 8, 11, 16, 32), so the
// instantiations build in parallel.
#include "tile_common.h"

#ifndef EKH_KNN_K
#error "compile with -DEKH_KNN_K=<list length>"
#endif

namespace ekh {

namespace {
template <int K, int QM, bool FULL> hipError_t knn_tile_launch(const KnnArgs &a, hipStream_t s) {
    constexpr int CB = knn_col_blocks(K, QM);
    constexpr int QT = kWaves * 16 * CB;
    const int64_t tail_q = (a.nq - a.body_q * QT + QT - 1) / QT;
    const int64_t groups = a.body_q + tail_q * a.splits;
    if (a.body_q < 0 || tail_q < 0 || a.splits < 1 || groups > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((knn_tile_kernel<K, QM, FULL>), dim3((unsigned)groups), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}
template <int K, int QM> hipError_t knn_tile_full(const KnnArgs &a, hipStream_t s) {
    return a.chunks == QM / 4 ? knn_tile_launch<K, QM, true>(a, s) : knn_tile_launch<K, QM, false>(a, s);
}
} // namespace

template <> hipError_t launch_knn_tile_k<EKH_KNN_K>(int QM, const KnnArgs &a, hipStream_t s) {
    switch (QM) {
    case 16: return knn_tile_full<EKH_KNN_K, 16>(a, s);
    case 32: return knn_tile_full<EKH_KNN_K, 32>(a, s);
    case 56: return knn_tile_full<EKH_KNN_K, 56>(a, s);
    case 64: return knn_tile_full<EKH_KNN_K, 64>(a, s);
    default: return hipErrorInvalidValue;
    }
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
