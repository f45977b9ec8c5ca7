// k_baseline.hip -- the two unfused steps the fused path replaces, kept as
// baselines for comparison on the same hardware:
//
//  * argmin over a materialised score matrix D [rows][K] (written by the
//    scores mode of the 16-bit assign kernel).  The pages (papernotes.org
//    notes "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", 核心问题
//    / 关键设计 1) identify the write and re-read of this N x K matrix as the
//    assign bottleneck that the fused kernel removes.
//  * the scatter-style update: every point adds its row into its centroid's
//    sum with d fp32 atomics and bumps the count.  The same notes (核心问题,
//    关键设计 2) identify the contention of these atomics on popular
//    centroids as the update bottleneck that the sort-inverse update removes.
#include "fk_internal.h"

namespace fk {
namespace {

constexpr int kBlk = 256;
constexpr int kRowsPerBlk = kBlk / kWave;

// Lexicographic (larger score, then lower index) merge.
__device__ inline void better(float& s, int32_t& k, float so, int32_t ko) {
    if (so > s || (so == s && ko < k)) {
        s = so;
        k = ko;
    }
}

// One wave per row of D: each lane walks its columns in ascending order
// (strict >, so the lowest index wins a tie), then the wave merges.
template <bool V4>
__global__ __launch_bounds__(kBlk) void k_argmin_rows(const float* __restrict__ D,
                                                     int32_t* __restrict__ labels, int64_t rows,
                                                     int64_t K) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * kRowsPerBlk + (threadIdx.x >> 6);
    if (r >= rows) return;
    const float* row = D + r * K;
    float best = -INFINITY;
    int32_t bi = 0x7fffffff;
    if constexpr (V4) {
        for (int64_t k0 = 4 * lane; k0 < K; k0 += 4 * kWave) {
            const floatx4 v = *reinterpret_cast<const floatx4*>(row + k0);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (v[q] > best) {
                    best = v[q];
                    bi = (int32_t)(k0 + q);
                }
        }
    } else {
        for (int64_t k = lane; k < K; k += kWave)
            if (row[k] > best) {
                best = row[k];
                bi = (int32_t)k;
            }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float so = __shfl_xor(best, o);
        const int32_t ko = __shfl_xor(bi, o);
        better(best, bi, so, ko);
    }
    // a row of NaN or -inf scores only: index 0, as the fused kernel
    if (lane == 0) labels[r] = bi == 0x7fffffff ? 0 : bi;
}

// One wave per point: d fp32 atomic adds into the sum row of its label and
// one into the count.  Labels outside [0, K) are skipped.
template <typename T>
__global__ __launch_bounds__(kBlk) void k_scatter_add(const T* __restrict__ X,
                                                     const int32_t* __restrict__ labels,
                                                     float* __restrict__ sums,
                                                     int32_t* __restrict__ counts, int64_t B,
                                                     int64_t N, int64_t K, int d) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * kRowsPerBlk + (threadIdx.x >> 6);
    if (i >= B * N) return;
    const int64_t b = i / N;
    const int32_t a = labels[i];
    if (a < 0 || a >= K) return;
    const T* x = X + i * d;
    float* s = sums + (b * K + a) * d;
    for (int j = lane; j < d; j += kWave) atomicAdd(s + j, (float)x[j]);
    if (lane == 0) atomicAdd(counts + b * K + a, 1);
}

}  // namespace

hipError_t launch_argmin_rows(const float* D, int32_t* labels, int64_t rows, int64_t K,
                              hipStream_t s) {
    const int64_t grid = (rows + kRowsPerBlk - 1) / kRowsPerBlk;
    if (K % 4 == 0 && (reinterpret_cast<uintptr_t>(D) & 15u) == 0)
        hipLaunchKernelGGL(k_argmin_rows<true>, dim3((unsigned)grid), dim3(kBlk), 0, s, D, labels,
                           rows, K);
    else
        hipLaunchKernelGGL(k_argmin_rows<false>, dim3((unsigned)grid), dim3(kBlk), 0, s, D, labels,
                           rows, K);
    return hipGetLastError();
}

hipError_t launch_scatter_add(int dtype, const void* X, const int32_t* labels, float* sums,
                              int32_t* counts, int64_t B, int64_t N, int64_t K, int d,
                              hipStream_t s) {
    const int64_t grid = (B * N + kRowsPerBlk - 1) / kRowsPerBlk;
    switch (dtype) {
        case FK_F16:
            hipLaunchKernelGGL(k_scatter_add<_Float16>, dim3((unsigned)grid), dim3(kBlk), 0, s,
                               static_cast<const _Float16*>(X), labels, sums, counts, B, N, K, d);
            break;
        case FK_BF16:
            hipLaunchKernelGGL(k_scatter_add<__bf16>, dim3((unsigned)grid), dim3(kBlk), 0, s,
                               static_cast<const __bf16*>(X), labels, sums, counts, B, N, K, d);
            break;
        default:
            hipLaunchKernelGGL(k_scatter_add<float>, dim3((unsigned)grid), dim3(kBlk), 0, s,
                               static_cast<const float*>(X), labels, sums, counts, B, N, K, d);
            break;
    }
    return hipGetLastError();
}

}  // namespace fk
