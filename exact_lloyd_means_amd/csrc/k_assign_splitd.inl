// k_assign_splitd.inl -- fused distance + argmin for long rows (split d).
//
// Same method as k_assign.inl (papernotes.org notes "Flash-KMeans: Fast and
// Memory-Efficient Exact K-Means", 关键设计 1: never store the N x K distance
// matrix, keep a running (min, argmin) per point) for rows too long to keep
// a point block in registers.  The 7minutos.es article on Flash-KMeans
// ("Usándolo") notes a separate path for large d; this is the MI355X one.
//
// Design: a workgroup of 8 waves owns 256 points of one problem and walks
// all K centroids in tiles of 256.  For each (point block, centroid tile)
// pair it accumulates the full dot products over d in 128-byte chunks: the
// point chunk [256 x 128 B] and the centroid chunk [256 x 128 B] are staged
// through registers into double-buffered LDS (16-byte slots XOR-swizzled by
// row, so the fragment reads are conflict-free).  Wave w computes points
// [128*(w%2), +128) x centroids [64*(w/2), +64) of the tile: 4 x 2 blocks of
// v_mfma_f32_32x32x16_{f16,bf16} (or 32x32x2_f32), 128 accumulators per
// lane, the centroid bias as the accumulator input of the first chunk.  After
// the last chunk each lane folds its 2 x 16 scores per point into a running
// (max score, lowest index); at the end the 4 waves x 2 half-waves holding
// the same point merge lexicographically through LDS.
#pragma once

#include <math.h>

#include "k_assign.inl"

namespace fk {
namespace {

constexpr int kSdWaves = 8;
constexpr int kSdP = 256;        // points per workgroup
constexpr int kSdK = 256;        // centroids per tile
constexpr int kSdRowB = 128;     // bytes of one row chunk
constexpr int kSdSlots = kSdRowB / 16;
constexpr int kSdStage = (kSdP + kSdK) * kSdRowB;  // LDS bytes per stage (X chunk + C chunk)

// LDS byte offset of 16-byte slot s of row r inside a [rows][128 B] chunk
__device__ inline int sd_slot(int r, int s) { return r * kSdRowB + ((s ^ (r & 7)) << 4); }

// VEC: d is a multiple of the 16-byte slot (slots load whole); else per element.
template <typename T, bool VEC, bool SMALLK>
__global__ __launch_bounds__(kSdWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_assign_splitd(const T* __restrict__ X, const T* __restrict__ C,
                     const float* __restrict__ bias, int32_t* __restrict__ labels,
                     float* __restrict__ min_dist, int64_t N, int64_t K, int d) {
    using M = Mfma<T>;
    constexpr int V = 16 / sizeof(T);         // elements per slot
    constexpr int EC = kSdRowB / sizeof(T);   // elements per row chunk
    constexpr int NT = kSdWaves * kWave;
    constexpr int LPT = (kSdP + kSdK) * kSdSlots / NT;  // 16-byte loads per thread per chunk

    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* s_stage = smem;                                          // [2][X chunk | C chunk]
    float* s_bias = reinterpret_cast<float*>(smem + 2 * kSdStage);  // [kSdK]
    float* s_best = s_bias + kSdK;                                  // [4][2][kSdP] merge
    int32_t* s_idx = reinterpret_cast<int32_t*>(s_best + 8 * kSdP);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int col = lane & 31;
    const int wp = wave & 1;           // point half of the tile
    const int wc = wave >> 1;          // centroid quarter of the tile
    const int64_t b = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * kSdP;
    const T* __restrict__ Xb = X + b * N * d;
    const T* __restrict__ Cb = C + b * K * d;
    const float* __restrict__ biasb = bias + b * K;
    const int K32 = (int)K;
    const int N32 = (int)N;
    const int nkt = (K32 + kSdK - 1) / kSdK;
    const int nch = (d + EC - 1) / EC;

    // thread tid moves, per chunk, LPT slots: rows [0, 256) are points,
    // rows [256, 512) centroids (row, slot) = (g / 8, g % 8), g = u*NT + tid
    auto load_slot = [&](int u, int kbase, int ch) -> u32x4 {
        const int g = u * NT + tid;
        const int r = g / kSdSlots;
        const int sl = g % kSdSlots;
        const int e0 = ch * EC + sl * V;
        if (r < kSdP) {
            const int row = min((int)p0 + r, N32 - 1);  // rows past N: any finite data
            return load_chunk<T, VEC>(Xb, row, N, d, e0);
        }
        const int k = kbase + (r - kSdP);
        return load_chunk<T, VEC>(Cb, SMALLK ? k : min(k, K32 - 1), K, d, e0);
    };
    auto store_slot = [&](int u, int buf, u32x4 v) {
        const int g = u * NT + tid;
        *reinterpret_cast<u32x4*>(s_stage + buf * kSdStage + sd_slot(g / kSdSlots, g % kSdSlots)) =
            v;
    };

    float best[4];
    int32_t bidx[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        best[cb] = -INFINITY;
        bidx[cb] = 0;
    }

    u32x4 pre[LPT];
    for (int kt = 0; kt < nkt; ++kt) {
        // tiles past the last start at K-256 and overlap the previous one: a
        // centroid seen twice cannot change a strict-">" running argmax
        const int kbase = SMALLK ? 0 : min(kt * kSdK, K32 - kSdK);
        // bias of this tile; rows past K (K < 256 only) can never win
        if (tid < kSdK) {
            const int k = kbase + tid;
            s_bias[tid] = k < K32 ? biasb[min(k, K32 - 1)] : -INFINITY;
        }
        floatx16 acc[2][4];
#pragma unroll
        for (int u = 0; u < LPT; ++u) pre[u] = load_slot(u, kbase, 0);
#pragma unroll
        for (int u = 0; u < LPT; ++u) store_slot(u, 0, pre[u]);
        __syncthreads();
        // bias vectors of this wave's two row blocks
        floatx16 bv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float* sb = s_bias + wc * 64 + rb * 32 + 4 * h;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const floatx4 v4 = *reinterpret_cast<const floatx4*>(sb + 8 * g);
                bv[rb][4 * g + 0] = v4[0];
                bv[rb][4 * g + 1] = v4[1];
                bv[rb][4 * g + 2] = v4[2];
                bv[rb][4 * g + 3] = v4[3];
            }
        }
        for (int ch = 0; ch < nch; ++ch) {
            const int buf = ch & 1;
            const bool more = ch + 1 < nch;
            if (more) {
#pragma unroll
                for (int u = 0; u < LPT; ++u) pre[u] = load_slot(u, kbase, ch + 1);
            }
            // 16-bit: raised issue priority for the chunk's matrix part,
            // normal for the staging stores and the barrier (2 % faster at
            // d = 1024 bf16; the fp32 form measured 1 % slower with it)
            if constexpr (sizeof(T) == 2) __builtin_amdgcn_s_setprio(1);
            const char* xs = s_stage + buf * kSdStage;
            const char* cs = xs + kSdP * kSdRowB;
#pragma unroll
            for (int s = 0; s < kSdSlots / 2; ++s) {
                u32x4 a[2], x[4];
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    a[rb] = *reinterpret_cast<const u32x4*>(cs + sd_slot(wc * 64 + rb * 32 + col, 2 * s + h));
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    x[cb] = *reinterpret_cast<const u32x4*>(xs + sd_slot(wp * 128 + cb * 32 + col, 2 * s + h));
#pragma unroll
                for (int e = 0; e < M::kSteps; ++e)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int cb = 0; cb < 4; ++cb)
                            acc[rb][cb] = M::step(a[rb], x[cb],
                                                  (ch == 0 && s == 0 && e == 0) ? bv[rb] : acc[rb][cb], e);
            }
            if constexpr (sizeof(T) == 2) __builtin_amdgcn_s_setprio(0);
            if (more) {
#pragma unroll
                for (int u = 0; u < LPT; ++u) store_slot(u, buf ^ 1, pre[u]);
            }
            __syncthreads();
        }
        // fold this tile's scores: rows ascend with (rb, r) inside a lane
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            float m = best[cb];
            int32_t rt = -1;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float sc = acc[rb][cb][r];
                    const bool keep = !(sc > m);
                    m = keep ? m : sc;
                    rt = keep ? rt : rb * 32 + 8 * (r >> 2) + (r & 3);
                }
            best[cb] = m;
            bidx[cb] = rt >= 0 ? kbase + wc * 64 + rt : bidx[cb];
        }
    }

    // ---- merge the 4 centroid quarters x 2 half-waves of every point
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int p = wp * 128 + cb * 32 + col;
        s_best[(wc * 2 + h) * kSdP + p] = best[cb];
        s_idx[(wc * 2 + h) * kSdP + p] = bidx[cb] + 4 * h;
    }
    __syncthreads();
    if (tid < kSdP) {
        const int p = tid;
        float sc = s_best[p];
        int32_t i = s_idx[p];
        for (int j = 1; j < 8; ++j) {
            const float so = s_best[j * kSdP + p];
            const int32_t io = s_idx[j * kSdP + p];
            if (so > sc || (so == sc && io < i)) {
                sc = so;
                i = io;
            }
        }
        const int64_t jn = p0 + p;
        if (jn < N) {
            labels[b * N + jn] = i;
            if (min_dist) {
                float xx = 0.f;
                const T* xr = Xb + jn * d;
                for (int e = 0; e < d; ++e) {
                    const float v = (float)xr[e];
                    xx = fmaf(v, v, xx);
                }
                min_dist[b * N + jn] = xx - 2.f * sc;
            }
        }
    }
}

constexpr size_t splitd_lds() {
    return 2 * (size_t)kSdStage + kSdK * sizeof(float) + 8 * kSdP * (sizeof(float) + sizeof(int32_t));
}

template <typename T>
hipError_t launch_assign_splitd(const void* X, const void* C, const float* bias, int32_t* labels,
                                float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                                hipStream_t s) {
    constexpr size_t lds = splitd_lds();
    static_assert(lds <= 160 * 1024, "LDS budget");
    constexpr int V = 16 / sizeof(T);
    const int variant = (K < kSdK ? 1 : 0) + (d % V == 0 ? 2 : 0);
    using Kern = void (*)(const T*, const T*, const float*, int32_t*, float*, int64_t, int64_t, int);
    const Kern kerns[4] = {k_assign_splitd<T, false, false>, k_assign_splitd<T, false, true>,
                           k_assign_splitd<T, true, false>, k_assign_splitd<T, true, true>};
    const Kern kern = kerns[variant];
    static LdsAttr attr[4];
    hipError_t e = ensure_lds(attr[variant], reinterpret_cast<const void*>(kern), (int)lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((N + kSdP - 1) / kSdP), (unsigned)B);
    hipLaunchKernelGGL(kern, grid, dim3(kSdWaves * kWave), lds, s, static_cast<const T*>(X),
                       static_cast<const T*>(C), bias, labels, min_dist, N, K, d);
    return hipGetLastError();
}

}  // namespace
}  // namespace fk
