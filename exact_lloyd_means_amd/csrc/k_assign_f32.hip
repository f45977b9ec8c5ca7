// k_assign_f32.hip -- instantiations of the fused assign kernels for float inputs.
#include "k_assign_splitd.inl"

namespace fk {
// Rows up to 128 dimensions keep each wave's points in registers for the
// whole K loop; longer rows stream d in chunks (split-d kernel).
hipError_t launch_assign_f32(const void* X, const void* C, const float* bias, int32_t* labels,
                         float* min_dist, int64_t B, int64_t N, int64_t K, int d, hipStream_t s) {
    if (d > 128)
        return launch_assign_splitd<float>(X, C, bias, labels, min_dist, B, N, K, d, s);
    return dispatch_assign<float>(X, C, bias, labels, min_dist, B, N, K, d, s);
}
}  // namespace fk
