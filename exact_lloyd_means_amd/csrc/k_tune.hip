// k_tune.hip -- every shape of the fp16 fused assign kernel that the
// register and LDS budgets admit, launchable one by one, so that the choice
// made by dispatch_assign16 (assign16_np, eight waves) can be checked
// against an exhaustive sweep.  Exact row widths d = 32 S only.
#include "k_assign16.inl"

namespace fk {
namespace {

template <int S, int NP, int W>
hipError_t tune_one(const void* X, const void* C, const float* bias, int32_t* labels, int64_t B,
                    int64_t N, int64_t K, int d, int64_t grid_wgs, hipStream_t s) {
    return launch_assign16_t<_Float16, S, NP, true, true, false, false, W>(
        X, C, bias, labels, nullptr, B, N, K, d, s, nullptr, grid_wgs);
}

template <int S, int W>
hipError_t tune_np(int np, const void* X, const void* C, const float* bias, int32_t* labels,
                   int64_t B, int64_t N, int64_t K, int d, int64_t grid_wgs, hipStream_t s) {
    switch (np) {
        case 1: return tune_one<S, 1, W>(X, C, bias, labels, B, N, K, d, grid_wgs, s);
        case 2: return tune_one<S, 2, W>(X, C, bias, labels, B, N, K, d, grid_wgs, s);
        case 4: return tune_one<S, 4, W>(X, C, bias, labels, B, N, K, d, grid_wgs, s);
        case 8: return tune_one<S, 8, W>(X, C, bias, labels, B, N, K, d, grid_wgs, s);
        default: return hipErrorInvalidValue;
    }
}

template <int S>
hipError_t tune_w(int np, int waves, const void* X, const void* C, const float* bias,
                  int32_t* labels, int64_t B, int64_t N, int64_t K, int d, int64_t grid_wgs,
                  hipStream_t s) {
    switch (waves) {
        case 2: return tune_np<S, 2>(np, X, C, bias, labels, B, N, K, d, grid_wgs, s);
        case 4: return tune_np<S, 4>(np, X, C, bias, labels, B, N, K, d, grid_wgs, s);
        case 8: return tune_np<S, 8>(np, X, C, bias, labels, B, N, K, d, grid_wgs, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_assign_variant(const void* X, const void* C, const float* bias, int32_t* labels,
                                 int64_t B, int64_t N, int64_t K, int d, int np, int waves,
                                 int64_t grid_wgs, hipStream_t s) {
    switch (d) {
        case 64: return tune_w<2>(np, waves, X, C, bias, labels, B, N, K, d, grid_wgs, s);
        case 128: return tune_w<4>(np, waves, X, C, bias, labels, B, N, K, d, grid_wgs, s);
        case 256: return tune_w<8>(np, waves, X, C, bias, labels, B, N, K, d, grid_wgs, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fk
