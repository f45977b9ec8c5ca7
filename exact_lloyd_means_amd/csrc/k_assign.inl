// k_assign.inl -- fused distance + running argmin on gfx950 matrix cores.
//
// Method: papernotes.org notes "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means", 关键设计 1 (FlashAssign).  Distances use the expansion
// |x - c|^2 = |x|^2 + |c|^2 - 2 x.c; per point a running minimum (m <- +inf)
// and index (a <- -1) are merged tile by tile with min / argmin, so the
// N x K distance matrix never leaves registers.
//
// MI355X design (not the pages' Hopper design):
//  * |x|^2 is constant per point and dropped from the comparison; the kernel
//    maximises the score s = x.c - |c|^2/2 (halving is exact), which orders
//    centroids exactly as -|x - c|^2 / 2 does.
//  * The centroid bias -|c|^2/2 enters as the accumulator input of the first
//    MFMA of every tile, so the epilogue is only compare + 2 selects.
//  * v_mfma_f32_32x32x16_{f16,bf16} (fp32 accumulate) or
//    v_mfma_f32_32x32x2_f32.  Rows of the 32x32 product are centroids,
//    columns are points, so each lane's 16 accumulators belong to one point
//    and the running (max, argmax) stays in that lane across all K tiles;
//    the two half-waves holding the same point merge once at the end.
//  * The contraction index is permuted: lane half h holds dimensions
//    [h*HR, (h+1)*HR) of its point, 16 bytes per MFMA step.  The same
//    permutation is applied to the centroid operand, so the dot product is
//    unchanged and each lane reads one contiguous half row.
//  * X rows of a wave stay in VGPRs for the whole K loop; centroid tiles of
//    32 rows stream HBM/L2 -> registers -> LDS, double buffered, one barrier
//    per tile.
//  * Exact tie rule: within a lane rows are visited in ascending index and a
//    row replaces the best only when strictly larger; half-waves merge
//    lexicographically on (score, index).  Padded centroid rows carry a
//    -inf bias and can never win.
#pragma once

#include <math.h>

#include "fk_internal.h"

namespace fk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
    static constexpr int kSteps = 1;  // MFMA steps per 16-byte chunk
    __device__ static inline floatx16 step(u32x4 a, u32x4 b, floatx16 c, int) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
    __device__ static inline float sumsq(u32x4 v) {
        half8 h = __builtin_bit_cast(half8, v);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf((float)h[e], (float)h[e], s);
        return s;
    }
};

template <>
struct Mfma<__bf16> {
    static constexpr int kSteps = 1;
    __device__ static inline floatx16 step(u32x4 a, u32x4 b, floatx16 c, int) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static inline float sumsq(u32x4 v) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo = __uint_as_float(v[e] << 16);
            float hi = __uint_as_float(v[e] & 0xffff0000u);
            s = fmaf(lo, lo, s);
            s = fmaf(hi, hi, s);
        }
        return s;
    }
};

template <>
struct Mfma<float> {
    static constexpr int kSteps = 4;
    __device__ static inline floatx16 step(u32x4 a, u32x4 b, floatx16 c, int e) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]),
                                                    c, 0, 0, 0);
    }
    __device__ static inline float sumsq(u32x4 v) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(__uint_as_float(v[e]), __uint_as_float(v[e]), s);
        return s;
    }
};

constexpr int kAssignWaves = 4;
constexpr int kAssignBK = 32;  // centroids per tile (one MFMA row block)

// Loads 16 bytes (V elements) of row `row` starting at element e0; elements
// at or beyond d, and rows at or beyond `rows`, read as zero.
template <typename T, bool VEC>
__device__ inline u32x4 load_chunk(const T* __restrict__ base, int64_t row, int64_t rows, int d,
                                   int e0) {
    constexpr int V = 16 / sizeof(T);
    u32x4 out = {0u, 0u, 0u, 0u};
    if (row >= rows) return out;
    const T* p = base + row * (int64_t)d;
    if constexpr (VEC) {
        if (e0 < d) out = *reinterpret_cast<const u32x4*>(p + e0);
    } else {
        T tmp[V];
#pragma unroll
        for (int e = 0; e < V; ++e) tmp[e] = (e0 + e < d) ? p[e0 + e] : (T)0;
        __builtin_memcpy(&out, tmp, 16);
    }
    return out;
}

// Q  = 16-byte chunks per half row (HR = Q * 16 / sizeof(T) dimensions),
// NB = 32-point column blocks held by each wave.
template <typename T, int Q, int NB, bool VEC>
__global__ __launch_bounds__(kAssignWaves * kWave) void k_assign(
    const T* __restrict__ X, const T* __restrict__ C, const float* __restrict__ bias,
    int32_t* __restrict__ labels, float* __restrict__ min_dist, int64_t N, int64_t K, int d) {
    using M = Mfma<T>;
    constexpr int V = 16 / sizeof(T);
    constexpr int HR = Q * V;                          // dimensions per half row
    constexpr int ROWB = 2 * Q * 16 + 16;              // LDS bytes per centroid row (padded)
    constexpr int TILEB = kAssignBK * ROWB;
    constexpr int CHUNKS = kAssignBK * 2 * Q;          // 16-byte chunks per tile
    constexpr int PER = (CHUNKS + kAssignWaves * kWave - 1) / (kAssignWaves * kWave);
    constexpr int PTS = kAssignWaves * NB * 32;        // points per workgroup

    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* s_tile = smem;                                            // [2][TILEB]
    float* s_bias = reinterpret_cast<float*>(smem + 2 * TILEB);     // [2][BK]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int col = lane & 31;
    const int64_t b = blockIdx.y;
    const T* __restrict__ Xb = X + b * N * d;
    const T* __restrict__ Cb = C + b * K * d;
    const float* __restrict__ biasb = bias + b * K;
    const int64_t pbase = (int64_t)blockIdx.x * PTS + (int64_t)wave * NB * 32;

    // ---- points of this wave: resident for the whole K loop
    u32x4 xf[NB][Q];
    float xsq[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        xsq[nb] = 0.f;
        const int64_t j = pbase + nb * 32 + col;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            xf[nb][q] = load_chunk<T, VEC>(Xb, j, N, d, h * HR + q * V);
            if (min_dist) xsq[nb] += M::sumsq(xf[nb][q]);
        }
    }

    // ---- centroid tile staging (registers -> LDS)
    u32x4 pre[PER];
    float pre_bias = 0.f;
    auto gload = [&](int64_t tbase) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = tid + u * kAssignWaves * kWave;
            if (c < CHUNKS) {
                const int r = c / (2 * Q);
                const int cc = c % (2 * Q);
                pre[u] = load_chunk<T, VEC>(Cb, tbase + r, K, d, cc * V);
            }
        }
        if (tid < kAssignBK) pre_bias = (tbase + tid < K) ? biasb[tbase + tid] : -INFINITY;
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = tid + u * kAssignWaves * kWave;
            if (c < CHUNKS) {
                const int r = c / (2 * Q);
                const int cc = c % (2 * Q);
                *reinterpret_cast<u32x4*>(s_tile + buf * TILEB + r * ROWB + cc * 16) = pre[u];
            }
        }
        if (tid < kAssignBK) s_bias[buf * kAssignBK + tid] = pre_bias;
    };

    float best[NB];
    int32_t bidx[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        best[nb] = -INFINITY;
        bidx[nb] = 0;
    }

    const int64_t ntiles = (K + kAssignBK - 1) / kAssignBK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t t = 0; t < ntiles; ++t) {
        const int buf = (int)(t & 1);
        if (t + 1 < ntiles) gload((t + 1) * kAssignBK);

        // bias of rows 8g + 4h + i (g = 0..3, i = 0..3): the accumulator rows of this lane
        floatx16 bv;
        const float* sb = s_bias + buf * kAssignBK + 4 * h;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const floatx4 v4 = *reinterpret_cast<const floatx4*>(sb + 8 * g);
            bv[4 * g + 0] = v4[0];
            bv[4 * g + 1] = v4[1];
            bv[4 * g + 2] = v4[2];
            bv[4 * g + 3] = v4[3];
        }

        floatx16 acc[NB];
        const char* arow = s_tile + buf * TILEB + col * ROWB + h * Q * 16;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(arow + q * 16);
#pragma unroll
            for (int e = 0; e < M::kSteps; ++e) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = M::step(a, xf[nb][q], (q == 0 && e == 0) ? bv : acc[nb], e);
            }
        }

        // epilogue: running (max score, lowest index); rows ascend with r
        const int32_t kb = (int32_t)(t * kAssignBK);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float s = acc[nb][r];
                const bool better = s > best[nb];
                best[nb] = better ? s : best[nb];
                bidx[nb] = better ? kb + 8 * (r >> 2) + (r & 3) : bidx[nb];
            }
        }

        if (t + 1 < ntiles) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- merge the two half-waves that hold the same point; write the label
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        float s = best[nb];
        int32_t i = bidx[nb] + 4 * h;
        const float so = __shfl_xor(s, 32);
        const int32_t io = __shfl_xor(i, 32);
        if (so > s || (so == s && io < i)) {
            s = so;
            i = io;
        }
        const float xx = xsq[nb] + __shfl_xor(xsq[nb], 32);
        const int64_t j = pbase + nb * 32 + col;
        if (h == 0 && j < N) {
            labels[b * N + j] = i;
            if (min_dist) min_dist[b * N + j] = xx - 2.f * s;
        }
    }
}

template <typename T, int Q, int NB, bool VEC>
hipError_t launch_assign_t(const void* X, const void* C, const float* bias, int32_t* labels,
                           float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                           hipStream_t s) {
    constexpr int ROWB = 2 * Q * 16 + 16;
    constexpr size_t lds = 2 * (size_t)kAssignBK * ROWB + 2 * kAssignBK * sizeof(float);
    constexpr int PTS = kAssignWaves * NB * 32;
    auto kern = k_assign<T, Q, NB, VEC>;
    static bool attr_set = false;  // one attribute call per instantiation and process
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid((unsigned)((N + PTS - 1) / PTS), (unsigned)B);
    hipLaunchKernelGGL(kern, grid, dim3(kAssignWaves * kWave), lds, s,
                       static_cast<const T*>(X), static_cast<const T*>(C), bias, labels, min_dist,
                       N, K, d);
    return hipGetLastError();
}

// Chooses Q (a power of two covering d) and the number of point blocks per
// wave that keeps X resident in VGPRs.
template <typename T>
hipError_t dispatch_assign(const void* X, const void* C, const float* bias, int32_t* labels,
                           float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                           hipStream_t s) {
    constexpr int V = 16 / sizeof(T);
    const int need = (d + 2 * V - 1) / (2 * V);  // chunks per half row
    const bool vec = (d % V) == 0;
#define FK_ASSIGN_CASE(QQ, NBB)                                                               \
    if (need <= QQ)                                                                           \
        return vec ? launch_assign_t<T, QQ, NBB, true>(X, C, bias, labels, min_dist, B, N, K, \
                                                       d, s)                                  \
                   : launch_assign_t<T, QQ, NBB, false>(X, C, bias, labels, min_dist, B, N,   \
                                                        K, d, s);
    FK_ASSIGN_CASE(1, 4)
    FK_ASSIGN_CASE(2, 4)
    FK_ASSIGN_CASE(4, 4)
    FK_ASSIGN_CASE(8, 4)
    FK_ASSIGN_CASE(16, 2)
    FK_ASSIGN_CASE(32, 1)
#undef FK_ASSIGN_CASE
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace fk
