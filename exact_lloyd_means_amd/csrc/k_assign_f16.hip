// k_assign_f16.hip -- instantiations of the fused assign kernels for _Float16 inputs.
#include "k_assign16.inl"
#include "k_assign_splitd.inl"

namespace fk {
// Rows up to 256 dimensions keep each wave's points in registers for the
// whole K loop (16x16x32 matrix instructions); longer rows, and rows of
// 129-256 dimensions that are not whole 16-byte chunks, stream d in chunks
// (split-d kernel; assign16_resident).
hipError_t launch_assign_f16(const void* X, const void* C, const float* bias, int32_t* labels,
                         float* min_dist, int64_t B, int64_t N, int64_t K, int d, hipStream_t s) {
    if (!assign16_resident(d))
        return launch_assign_splitd<_Float16>(X, C, bias, labels, min_dist, B, N, K, d, s);
    return dispatch_assign16<_Float16>(X, C, bias, labels, min_dist, B, N, K, d, s);
}
// Scores mode of the same kernel (d <= 256): every x.c + bias into D.
hipError_t launch_scores_f16(const void* X, const void* C, const float* bias, float* D, int64_t B,
                          int64_t N, int64_t K, int d, hipStream_t s) {
    return dispatch_scores16<_Float16>(X, C, bias, D, B, N, K, d, s);
}
}  // namespace fk
