// k_update.hip -- sort-inverse centroid update on gfx950, and small helpers.
//
// Method: papernotes.org notes "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means", 关键设计 2 (Sort-Inverse Update): argsort the 1-D label vector so
// equal labels form contiguous segments, split fixed-length runs of sorted
// positions into same-label pieces [u, v), gather the X rows named by the
// sorted indices (X itself never moves), reduce each piece on chip and issue
// one atomic add per piece: O((K + N/B_N) d) atomics instead of O(N d).
//
// MI355X design:
//  * The argsort is a counting sort, since keys are small integers in [0, K):
//    histogram (LDS-privatised) -> exclusive scan -> scatter, where each
//    workgroup reserves one range per label with a single global atomic and
//    ranks its elements inside that range with LDS atomics.  Order inside a
//    segment is unspecified; the grouping is exact.
//  * The gather-reduce gives every wave a fixed run of sorted positions.  The
//    segment walk is wave-uniform (indices and offsets come through the
//    scalar unit), lanes split the d dimensions of each row, rows are loaded
//    several at a time for memory-level parallelism, and a piece ends with
//    one row of fp32 atomic adds.
//  * Finalize divides by the exact integer count (IEEE fp32 division), keeps
//    empty centroids bit for bit, writes the round-to-nearest-even copy in
//    the input dtype with its |c|^2 bias for the next assignment, tracks the
//    largest squared centroid move and clears the sums for the next call.
#include <math.h>

#include "fk_internal.h"

namespace fk {
namespace {

constexpr int kBlock = 256;
constexpr int kSortTile = 4096;          // labels per histogram / scatter workgroup
constexpr int64_t kLdsBinsMax = 16384;   // LDS-privatised bins (64 KiB)
constexpr int kSegChunk = 64;            // sorted positions per wave in the gather-reduce
constexpr int kSegUnroll = 8;            // rows in flight per wave

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T>
__device__ inline float to_f32(T v) {
    return (float)v;
}

// ---------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void k_add_i32(int32_t* __restrict__ dst, const int32_t* __restrict__ src, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] += src[i];
}

// bias[row] = -0.5 * sum_j C[row][j]^2 in fp32 (one wave per centroid row)
template <typename T>
__global__ __launch_bounds__(kBlock) void k_centroid_bias(const T* __restrict__ C,
                                                          float* __restrict__ bias, int64_t rows,
                                                          int d) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const T* c = C + row * d;
    float s = 0.f;
    for (int j = lane; j < d; j += kWave) {
        const float v = to_f32(c[j]);
        s = fmaf(v, v, s);
    }
    s = wave_sum(s);
    if (lane == 0) bias[row] = -0.5f * s;
}

// lowp = RNE(C) in the input dtype, bias from the rounded values
template <typename T>
__global__ __launch_bounds__(kBlock) void k_prepare(const float* __restrict__ C, T* __restrict__ lowp,
                                                    float* __restrict__ bias, int64_t rows, int d) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    if (row >= rows) return;
    float s = 0.f;
    for (int j = lane; j < d; j += kWave) {
        const T q = (T)C[row * d + j];
        lowp[row * d + j] = q;
        const float v = to_f32(q);
        s = fmaf(v, v, s);
    }
    s = wave_sum(s);
    if (lane == 0) bias[row] = -0.5f * s;
}

// ---------------------------------------------------------------------------
// counts[b][k] += #{i in tile : labels[b][i] == k}; out-of-range labels are
// counted in flags[0] and skipped.
__global__ __launch_bounds__(kBlock) void k_histogram(const int32_t* __restrict__ labels,
                                                      int32_t* __restrict__ counts,
                                                      uint32_t* __restrict__ flags, int64_t N,
                                                      int64_t K, int use_lds) {
    extern __shared__ int32_t s_hist[];
    const int64_t b = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * kSortTile;
    const int64_t i1 = min(i0 + (int64_t)kSortTile, N);
    const int32_t* lab = labels + b * N;
    int32_t* cnt = counts + b * K;
    uint32_t bad = 0;
    if (use_lds) {
        for (int64_t k = threadIdx.x; k < K; k += kBlock) s_hist[k] = 0;
        __syncthreads();
        for (int64_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
            const int32_t a = lab[i];
            if (a >= 0 && a < K)
                atomicAdd(&s_hist[a], 1);
            else
                ++bad;
        }
        __syncthreads();
        for (int64_t k = threadIdx.x; k < K; k += kBlock) {
            const int32_t v = s_hist[k];
            if (v) atomicAdd(&cnt[k], v);
        }
    } else {
        for (int64_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
            const int32_t a = lab[i];
            if (a >= 0 && a < K)
                atomicAdd(&cnt[a], 1);
            else
                ++bad;
        }
    }
    if (bad) atomicAdd(&flags[0], bad);
}

// offsets[b][k] = sum_{k' < k} counts[b][k'], offsets[b][K] = total; cursor = offsets
__global__ __launch_bounds__(kBlock) void k_scan(const int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ cursor, int64_t K) {
    __shared__ int32_t s[kBlock];
    const int64_t b = blockIdx.x;
    const int32_t* c = counts + b * K;
    int32_t* off = offsets + b * (K + 1);
    int32_t* cur = cursor + b * K;
    const int64_t per = (K + kBlock - 1) / kBlock;
    const int64_t k0 = min((int64_t)threadIdx.x * per, K);
    const int64_t k1 = min(k0 + per, K);
    int32_t local = 0;
    for (int64_t k = k0; k < k1; ++k) local += c[k];
    s[threadIdx.x] = local;
    __syncthreads();
    for (int o = 1; o < kBlock; o <<= 1) {
        const int32_t v = threadIdx.x >= o ? s[threadIdx.x - o] : 0;
        __syncthreads();
        s[threadIdx.x] += v;
        __syncthreads();
    }
    int32_t run = s[threadIdx.x] - local;
    for (int64_t k = k0; k < k1; ++k) {
        off[k] = run;
        cur[k] = run;
        run += c[k];
    }
    if (threadIdx.x == kBlock - 1) off[K] = s[kBlock - 1];
}

// sorted_idx[b][pos] = i with pos inside label a_i's segment; sorted_lab
// (optional) receives the label at each sorted position
__global__ __launch_bounds__(kBlock) void k_scatter(const int32_t* __restrict__ labels,
                                                    int32_t* __restrict__ cursor,
                                                    int32_t* __restrict__ sorted_idx,
                                                    int32_t* __restrict__ sorted_lab, int64_t N,
                                                    int64_t K, int use_lds) {
    extern __shared__ int32_t s_base[];
    const int64_t b = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * kSortTile;
    const int64_t i1 = min(i0 + (int64_t)kSortTile, N);
    const int32_t* lab = labels + b * N;
    int32_t* cur = cursor + b * K;
    int32_t* out = sorted_idx + b * N;
    int32_t* olab = sorted_lab ? sorted_lab + b * N : nullptr;
    if (use_lds) {
        for (int64_t k = threadIdx.x; k < K; k += kBlock) s_base[k] = 0;
        __syncthreads();
        for (int64_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
            const int32_t a = lab[i];
            if (a >= 0 && a < K) atomicAdd(&s_base[a], 1);
        }
        __syncthreads();
        // one global reservation per label present in this tile
        for (int64_t k = threadIdx.x; k < K; k += kBlock) {
            const int32_t v = s_base[k];
            if (v) s_base[k] = atomicAdd(&cur[k], v);
        }
        __syncthreads();
        for (int64_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
            const int32_t a = lab[i];
            if (a >= 0 && a < K) {
                const int32_t pos = atomicAdd(&s_base[a], 1);
                out[pos] = (int32_t)i;
                if (olab) olab[pos] = a;
            }
        }
    } else {
        for (int64_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
            const int32_t a = lab[i];
            if (a >= 0 && a < K) {
                const int32_t pos = atomicAdd(&cur[a], 1);
                out[pos] = (int32_t)i;
                if (olab) olab[pos] = a;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The EPL stored elements of row `row` owned by this lane (dims e0..e0+EPL-1);
// dims at or beyond d read as zero.
template <typename T, int EPL>
struct RowPart {
    T v[EPL];
};
template <typename T, int EPL, bool VEC>
__device__ inline RowPart<T, EPL> load_row_part(const T* __restrict__ base, int64_t row, int d,
                                                int e0) {
    const T* p = base + row * (int64_t)d + e0;
    RowPart<T, EPL> r;
    if constexpr (VEC) {
        __builtin_memcpy(r.v, __builtin_assume_aligned(p, EPL * sizeof(T) >= 16 ? 16 : EPL * sizeof(T)),
                         sizeof(r.v));
    } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) r.v[e] = (e0 + e < d) ? p[e] : (T)0;
    }
    return r;
}

// Rows gathered per batch so that the loaded values fit in about 64 VGPRs.
template <typename T, int EPL>
constexpr int seg_batch() {
    constexpr int regs = (EPL * (int)sizeof(T) + 3) / 4;
    return regs >= 64 ? 1 : 64 / regs;
}

// Each wave reduces kSegChunk = 64 consecutive sorted positions.  Its 64
// point indices and labels arrive with one coalesced load (one per lane);
// row addresses are then read lane by lane (readlane, no memory latency),
// a batch of rows is loaded back to back, and the rows are added in order,
// closing a piece with one row of atomic adds whenever the label changes.
// sums must be zero on entry (or hold earlier partial sums to add to).
template <typename T, int EPL, bool VEC>
__global__ __launch_bounds__(kBlock) void k_segment_sums(const T* __restrict__ X,
                                                         const int32_t* __restrict__ sorted_idx,
                                                         const int32_t* __restrict__ sorted_lab,
                                                         const int32_t* __restrict__ offsets,
                                                         float* __restrict__ sums, int64_t N,
                                                         int64_t K, int d) {
    static_assert(kSegChunk == kWave, "one sorted position per lane");
    constexpr int RB = seg_batch<T, EPL>();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t b = blockIdx.y;
    // positions past offsets[K] exist only when out-of-range labels were skipped
    const int64_t total = offsets[b * (K + 1) + K];
    const int64_t p0 = ((int64_t)blockIdx.x * (kBlock / kWave) + wave) * kSegChunk;
    if (p0 >= total) return;
    const int n = (int)min((int64_t)kSegChunk, total - p0);  // positions of this wave
    const T* __restrict__ Xb = X + b * N * d;
    float* __restrict__ Sb = sums + b * K * d;
    const int64_t q = p0 + min(lane, n - 1);
    const int32_t vidx = sorted_idx[b * N + q];
    const int32_t vlab = sorted_lab[b * N + q];

    const int e0 = lane * EPL;
    const bool active = e0 < d;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    int32_t cur = __builtin_amdgcn_readfirstlane(vlab);

    auto flush = [&](int32_t kk) {
        if (active) {
            float* dst = Sb + (int64_t)kk * d + e0;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                if (VEC || e0 + e < d) atomicAdd(dst + e, acc[e]);
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    };

#pragma unroll
    for (int base = 0; base < kSegChunk; base += RB) {
        if (base < n) {
            // all loads of the batch first, unconditionally, so they are in
            // flight together: positions past n re-read the last row and
            // lanes past d read the row start; neither is ever added
            RowPart<T, EPL> v[RB];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                const int32_t row = __builtin_amdgcn_readlane(vidx, base + u);
                v[u] = load_row_part<T, EPL, VEC>(Xb, row, d, active ? e0 : 0);
            }
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                if (base + u < n) {
                    const int32_t a = __builtin_amdgcn_readlane(vlab, base + u);
                    if (a != cur) {
                        flush(cur);
                        cur = a;
                    }
                    if (active) {
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[e] += to_f32(v[u].v[e]);
                    }
                }
            }
        }
    }
    flush(cur);
}

// ---------------------------------------------------------------------------
template <typename T, bool LOWP>
__global__ __launch_bounds__(kBlock) void k_finalize(float* __restrict__ sums,
                                                     const int32_t* __restrict__ counts,
                                                     const float* C_prev, float* C_next,
                                                     T* __restrict__ lowp,
                                                     float* __restrict__ bias,
                                                     uint32_t* __restrict__ move_max,
                                                     int64_t rows, int d) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int32_t n = counts[row];
    const float fn = (float)n;
    float cn = 0.f, mv = 0.f;
    for (int j = lane; j < d; j += kWave) {
        const int64_t o = row * d + j;
        const float prev = C_prev[o];
        const float c = n > 0 ? sums[o] / fn : prev;
        C_next[o] = c;
        sums[o] = 0.f;
        float cq = c;
        if constexpr (LOWP) {
            const T q = (T)c;
            if (lowp) lowp[o] = q;
            cq = to_f32(q);
        }
        cn = fmaf(cq, cq, cn);
        const float m = c - prev;
        mv = fmaf(m, m, mv);
    }
    if (bias) {
        cn = wave_sum(cn);
        if (lane == 0) bias[row] = -0.5f * cn;
    }
    if (move_max) {
        mv = wave_sum(mv);
        if (lane == 0) atomicMax(move_max, __float_as_uint(mv));
    }
}

inline unsigned grid_rows(int64_t rows) {
    return (unsigned)((rows + (kBlock / kWave) - 1) / (kBlock / kWave));
}

template <typename T>
hipError_t segment_sums_t(const void* X, const int32_t* sorted_idx, const int32_t* sorted_lab,
                          const int32_t* offsets, float* sums, int64_t B, int64_t N, int64_t K,
                          int d, hipStream_t s) {
    const int epl = (d + kWave - 1) / kWave;
    const dim3 grid((unsigned)((N + (int64_t)kSegChunk * (kBlock / kWave) - 1) /
                               ((int64_t)kSegChunk * (kBlock / kWave))),
                    (unsigned)B);
    const T* x = static_cast<const T*>(X);
#define FK_SEG_CASE(E)                                                                        \
    if (epl <= E) {                                                                           \
        if (d % E == 0)                                                                       \
            hipLaunchKernelGGL((k_segment_sums<T, E, true>), grid, dim3(kBlock), 0, s, x,     \
                               sorted_idx, sorted_lab, offsets, sums, N, K, d);               \
        else                                                                                  \
            hipLaunchKernelGGL((k_segment_sums<T, E, false>), grid, dim3(kBlock), 0, s, x,    \
                               sorted_idx, sorted_lab, offsets, sums, N, K, d);               \
        return hipGetLastError();                                                             \
    }
    FK_SEG_CASE(1)
    FK_SEG_CASE(2)
    FK_SEG_CASE(4)
    FK_SEG_CASE(8)
    FK_SEG_CASE(16)
#undef FK_SEG_CASE
    return hipErrorInvalidValue;
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_fill_u32(uint32_t* ptr, int64_t n, uint32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = min((n + kBlock - 1) / kBlock, (int64_t)4096);
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(kBlock), 0, s, ptr, n, value);
    return hipGetLastError();
}

hipError_t launch_add_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = min((n + kBlock - 1) / kBlock, (int64_t)1024);
    hipLaunchKernelGGL(k_add_i32, dim3((unsigned)blocks), dim3(kBlock), 0, s, dst, src, n);
    return hipGetLastError();
}

hipError_t launch_centroid_bias(int dtype, const void* C, float* bias, int64_t rows, int d,
                                hipStream_t s) {
    const dim3 grid(grid_rows(rows));
    switch (dtype) {
        case FK_F32:
            hipLaunchKernelGGL(k_centroid_bias<float>, grid, dim3(kBlock), 0, s,
                               static_cast<const float*>(C), bias, rows, d);
            break;
        case FK_F16:
            hipLaunchKernelGGL(k_centroid_bias<_Float16>, grid, dim3(kBlock), 0, s,
                               static_cast<const _Float16*>(C), bias, rows, d);
            break;
        default:
            hipLaunchKernelGGL(k_centroid_bias<__bf16>, grid, dim3(kBlock), 0, s,
                               static_cast<const __bf16*>(C), bias, rows, d);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_prepare(int dtype, const float* C, void* lowp, float* bias, int64_t rows, int d,
                          hipStream_t s) {
    const dim3 grid(grid_rows(rows));
    if (dtype == FK_F16)
        hipLaunchKernelGGL(k_prepare<_Float16>, grid, dim3(kBlock), 0, s, C,
                           static_cast<_Float16*>(lowp), bias, rows, d);
    else if (dtype == FK_BF16)
        hipLaunchKernelGGL(k_prepare<__bf16>, grid, dim3(kBlock), 0, s, C,
                           static_cast<__bf16*>(lowp), bias, rows, d);
    else
        return launch_centroid_bias(FK_F32, C, bias, rows, d, s);
    return hipGetLastError();
}

hipError_t launch_histogram(const int32_t* labels, int32_t* counts, uint32_t* flags, int64_t B,
                            int64_t N, int64_t K, hipStream_t s) {
    const int use_lds = K <= kLdsBinsMax;
    const size_t lds = use_lds ? (size_t)K * sizeof(int32_t) : 0;
    const dim3 grid((unsigned)((N + kSortTile - 1) / kSortTile), (unsigned)B);
    hipLaunchKernelGGL(k_histogram, grid, dim3(kBlock), lds, s, labels, counts, flags, N, K,
                       use_lds);
    return hipGetLastError();
}

hipError_t launch_scan(const int32_t* counts, int32_t* offsets, int32_t* cursor, int64_t B,
                       int64_t K, hipStream_t s) {
    hipLaunchKernelGGL(k_scan, dim3((unsigned)B), dim3(kBlock), 0, s, counts, offsets, cursor, K);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* labels, int32_t* cursor, int32_t* sorted_idx,
                          int32_t* sorted_lab, int64_t B, int64_t N, int64_t K, hipStream_t s) {
    const int use_lds = K <= kLdsBinsMax;
    const size_t lds = use_lds ? (size_t)K * sizeof(int32_t) : 0;
    const dim3 grid((unsigned)((N + kSortTile - 1) / kSortTile), (unsigned)B);
    hipLaunchKernelGGL(k_scatter, grid, dim3(kBlock), lds, s, labels, cursor, sorted_idx,
                       sorted_lab, N, K, use_lds);
    return hipGetLastError();
}

hipError_t launch_segment_sums(int dtype, const void* X, const int32_t* sorted_idx,
                               const int32_t* sorted_lab, const int32_t* offsets, float* sums,
                               int64_t B, int64_t N, int64_t K, int d, hipStream_t s) {
    switch (dtype) {
        case FK_F32:
            return segment_sums_t<float>(X, sorted_idx, sorted_lab, offsets, sums, B, N, K, d, s);
        case FK_F16:
            return segment_sums_t<_Float16>(X, sorted_idx, sorted_lab, offsets, sums, B, N, K, d, s);
        default:
            return segment_sums_t<__bf16>(X, sorted_idx, sorted_lab, offsets, sums, B, N, K, d, s);
    }
}

hipError_t launch_finalize(int dtype, float* sums, const int32_t* counts, const float* C_prev,
                           float* C_next, void* lowp, float* bias, uint32_t* move_max,
                           int64_t rows, int d, hipStream_t s) {
    const dim3 grid(grid_rows(rows));
    if (dtype == FK_F16)
        hipLaunchKernelGGL((k_finalize<_Float16, true>), grid, dim3(kBlock), 0, s, sums, counts,
                           C_prev, C_next, static_cast<_Float16*>(lowp), bias, move_max, rows, d);
    else if (dtype == FK_BF16)
        hipLaunchKernelGGL((k_finalize<__bf16, true>), grid, dim3(kBlock), 0, s, sums, counts,
                           C_prev, C_next, static_cast<__bf16*>(lowp), bias, move_max, rows, d);
    else
        hipLaunchKernelGGL((k_finalize<float, false>), grid, dim3(kBlock), 0, s, sums, counts,
                           C_prev, C_next, static_cast<float*>(nullptr), bias, move_max, rows, d);
    return hipGetLastError();
}

}  // namespace fk
