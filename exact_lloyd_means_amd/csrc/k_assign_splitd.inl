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
// point chunk [256 x 128 B] and the centroid chunk [256 x 128 B] reach
// double-buffered LDS (16-byte slots XOR-swizzled by row, so the fragment
// reads are conflict-free).  Wave w computes points [128*(w%2), +128) x
// centroids [64*(w/2), +64) of the tile: 8 x 4 blocks of
// v_mfma_f32_16x16x32_{f16,bf16} (fp32 and register staging: 4 x 2 blocks
// of the 32x32 forms), 128 accumulators per lane, the centroid bias as the
// accumulators' start.  After the last chunk each lane folds its scores of every
// point it holds into a running (max score, lowest index); at the end the
// candidates of each point (row groups, centroid quarters) merge
// lexicographically.
#pragma once

#include <math.h>

#include "k_assign16.inl"

namespace fk {
namespace {

constexpr int kSdWaves = 8;
constexpr int kSdP = 256;        // points per workgroup
constexpr int kSdK = 256;        // centroids per tile
constexpr int kSdRowB = 128;     // bytes of one row chunk
constexpr int kSdSlots = kSdRowB / 16;
constexpr int kSdStage = (kSdP + kSdK) * kSdRowB;  // LDS bytes per stage (X chunk + C chunk)

// LDS byte offset of 16-byte slot s of row r inside a [rows][128 B] chunk.
// Two 128-byte rows share a 256-byte line of the 64 banks (row parity picks
// the half); XORing the slot with (r / 2) % 8 gives each of 16 consecutive
// rows read at one slot its own 16-byte bank group, so a fragment read (16
// lanes per pass, consecutive rows) is conflict-free.
__device__ inline int sd_slot(int r, int s) { return r * kSdRowB + ((s ^ ((r >> 1) & 7)) << 4); }

// VEC: d is a multiple of the 16-byte slot (slots load whole); else per element.
// DMA (whole 128-byte chunks, K >= 256, each problem's rows under 4 GiB):
// the chunks reach LDS by direct global-to-LDS loads instead of through
// registers.  Wave w's load u fills LDS bytes [(8 u + w) KiB, +1 KiB) of the
// stage: rows 8 (8 u + w) .. + 7, lane i taking physical slot i % 8 of row
// (8 u + w) 8 + i / 8, i.e. the row's logical slot (i % 8) ^ ((row / 2) % 8),
// so the swizzled layout the fragment reads expect comes out of the linear
// lane-order writes of the load.
// U (rows that are not whole slots, !VEC): 8 or 4 = rows read in units of
// that many bytes (the widest dividing the row stride); 0 = element by
// element.
template <typename T, bool VEC, bool SMALLK, bool DMA, int U = 0>
__global__ __launch_bounds__(kSdWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_assign_splitd(const T* __restrict__ X, const T* __restrict__ C,
                     const float* __restrict__ bias, int32_t* __restrict__ labels,
                     float* __restrict__ min_dist, int64_t N, int64_t K, int d) {
    static_assert(!DMA || (VEC && !SMALLK), "direct loads need whole slots and full tiles");
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
        auto ld = [&](const T* base, int row, int64_t rows) -> u32x4 {
            if constexpr (!VEC && U > 0)
                return load_chunk_units<T, U>(base, row, rows, d, e0);
            else
                return load_chunk<T, VEC>(base, row, rows, d, e0);
        };
        if (r < kSdP) {
            const int row = min((int)p0 + r, N32 - 1);  // rows past N: any finite data
            return ld(Xb, row, N);
        }
        const int k = kbase + (r - kSdP);
        return ld(Cb, SMALLK ? k : min(k, K32 - 1), K);
    };
    auto store_slot = [&](int u, int buf, u32x4 v) {
        const int g = u * NT + tid;
        *reinterpret_cast<u32x4*>(s_stage + buf * kSdStage + sd_slot(g / kSdSlots, g % kSdSlots)) =
            v;
    };
    // direct loads: per lane, the row and the byte offset of its logical
    // slot inside a chunk; loads u < LPT / 2 fill point rows, the others
    // centroid rows (kSdP / 8 / kSdWaves = LPT / 2)
    static_assert(kSdP == kSdK && LPT == 8 && kSdSlots == 8, "direct-load layout");
    const uint32_t rowb = (uint32_t)d * (uint32_t)sizeof(T);
    uint32_t dma_row[LPT];  // point row (global) or centroid row within the tile
    // (row / 2) % 8 = (4 (wave % 2) + lane / 16) % 8: rows of load u start at
    // a multiple of 8 rows, 8 (8 u + wave)
    const uint32_t dma_slot = (uint32_t)(((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7)) * 16);
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
        const int r = (u * kSdWaves + wave) * 8 + (lane >> 3);
        dma_row[u] = r < kSdP ? (uint32_t)min((int)p0 + r, N32 - 1) : (uint32_t)(r - kSdP);
    }
    auto dma_chunk = [&](int kbase, int ch, int buf) {
        const uint32_t cho = (uint32_t)ch * kSdRowB + dma_slot;
        char* st = s_stage + buf * kSdStage;
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const uint32_t lds = (uint32_t)(uintptr_t)(st + (u * kSdWaves + wave) * 1024);
            if (u < LPT / 2)
                lds_dma16(Xb, dma_row[u] * rowb + cho, __builtin_amdgcn_readfirstlane(lds));
            else
                lds_dma16(Cb, ((uint32_t)kbase + dma_row[u]) * rowb + cho,
                          __builtin_amdgcn_readfirstlane(lds));
        }
    };

    // 16-bit inputs with direct loads use v_mfma_f32_16x16x32 (a quarter of
    // the accumulator registers per instruction, which sustains more flops
    // under the power limit than the 32x32x16 form): lane (g, c) = (lane / 16,
    // lane % 16) holds rows 4 g + i of a 16-centroid block for point column
    // c, so a wave's 128 x 64 scores are 8 point blocks x 4 centroid blocks
    // and each lane keeps one running (max, index) per point block.  fp32
    // and the register-staged forms (whose staging registers leave no room
    // for the 16x16 fragments) keep the 32x32 form: 4 point blocks of 32,
    // two half-waves per point.
    constexpr bool M16 = sizeof(T) == 2 && DMA;
    constexpr int NB = M16 ? 8 : 4;  // point blocks (running maxima) per lane
    const int g = lane >> 4, c16 = lane & 15;
    float best[NB];
    int32_t bidx[NB];
#pragma unroll
    for (int pb = 0; pb < NB; ++pb) {
        best[pb] = -INFINITY;
        bidx[pb] = 0;
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
        floatx4 acc16[4][8];
        if constexpr (DMA) {
            dma_chunk(kbase, 0, 0);
            wait_vm<0>();
        } else {
#pragma unroll
            for (int u = 0; u < LPT; ++u) pre[u] = load_slot(u, kbase, 0);
#pragma unroll
            for (int u = 0; u < LPT; ++u) store_slot(u, 0, pre[u]);
        }
        __syncthreads();
        // bias vectors of this wave's row blocks (the accumulators' rows)
        floatx16 bv[2];
        if constexpr (M16) {
            // (the accumulators start at the bias: nothing extra stays live
            // through the chunk loop)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const floatx4 b4 =
                    *reinterpret_cast<const floatx4*>(s_bias + wc * 64 + cb * 16 + 4 * g);
#pragma unroll
                for (int pb = 0; pb < 8; ++pb) acc16[cb][pb] = b4;
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const float* sb = s_bias + wc * 64 + rb * 32 + 4 * h;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const floatx4 v4 = *reinterpret_cast<const floatx4*>(sb + 8 * q);
                    bv[rb][4 * q + 0] = v4[0];
                    bv[rb][4 * q + 1] = v4[1];
                    bv[rb][4 * q + 2] = v4[2];
                    bv[rb][4 * q + 3] = v4[3];
                }
            }
        }
        for (int ch = 0; ch < nch; ++ch) {
            const int buf = ch & 1;
            const bool more = ch + 1 < nch;
            if (more) {
                // the other buffer was last read before the previous barrier
                if constexpr (DMA) {
                    dma_chunk(kbase, ch + 1, buf ^ 1);
                } else {
#pragma unroll
                    for (int u = 0; u < LPT; ++u) pre[u] = load_slot(u, kbase, ch + 1);
                }
            }
            // 16-bit: raised issue priority for the chunk's matrix part,
            // normal for the staging stores and the barrier (2 % faster at
            // d = 1024 bf16; the fp32 form measured 1 % slower with it)
            if constexpr (sizeof(T) == 2) __builtin_amdgcn_s_setprio(1);
            const char* xs = s_stage + buf * kSdStage;
            const char* cs = xs + kSdP * kSdRowB;
            if constexpr (M16) {
                // two k-steps of 32 per chunk: lane group g reads slot 4 ks + g
                // of its 16 centroid rows (A) and 16 point rows (B)
#pragma unroll
                for (int ks = 0; ks < kSdSlots / 4; ++ks) {
                    u32x4 a[4], x[8];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        a[cb] = *reinterpret_cast<const u32x4*>(
                            cs + sd_slot(wc * 64 + cb * 16 + c16, 4 * ks + g));
#pragma unroll
                    for (int pb = 0; pb < 8; ++pb)
                        x[pb] = *reinterpret_cast<const u32x4*>(
                            xs + sd_slot(wp * 128 + pb * 16 + c16, 4 * ks + g));
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                        for (int pb = 0; pb < 8; ++pb)
                            acc16[cb][pb] = Mfma16<T>::step(a[cb], x[pb], acc16[cb][pb]);
                }
            } else {
#pragma unroll
                for (int s = 0; s < kSdSlots / 2; ++s) {
                    u32x4 a[2], x[4];
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
                        a[rb] = *reinterpret_cast<const u32x4*>(
                            cs + sd_slot(wc * 64 + rb * 32 + col, 2 * s + h));
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        x[cb] = *reinterpret_cast<const u32x4*>(
                            xs + sd_slot(wp * 128 + cb * 32 + col, 2 * s + h));
#pragma unroll
                    for (int e = 0; e < M::kSteps; ++e)
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                            for (int cb = 0; cb < 4; ++cb)
                                acc[rb][cb] = M::step(
                                    a[rb], x[cb],
                                    (ch == 0 && s == 0 && e == 0) ? bv[rb] : acc[rb][cb], e);
                }
            }
            if constexpr (sizeof(T) == 2) __builtin_amdgcn_s_setprio(0);
            if (more) {
                if constexpr (DMA) {
                    wait_vm<0>();  // this wave's part of the next chunk has landed
                } else {
#pragma unroll
                    for (int u = 0; u < LPT; ++u) store_slot(u, buf ^ 1, pre[u]);
                }
            }
            __syncthreads();
        }
        // fold this tile's scores: rows ascend with (cb, i) (16-bit) or
        // (rb, r) (fp32) inside a lane
        if constexpr (M16) {
#pragma unroll
            for (int pb = 0; pb < 8; ++pb) {
                float m = best[pb];
                int32_t rt = -1;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float sc = acc16[cb][pb][i];
                        const bool keep = !(sc > m);
                        m = keep ? m : sc;
                        rt = keep ? rt : cb * 16 + 4 * g + i;
                    }
                best[pb] = m;
                bidx[pb] = rt >= 0 ? kbase + wc * 64 + rt : bidx[pb];
            }
        } else {
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
    }

    // ---- merge every point's candidates (lexicographic on (score, index)):
    // 16-bit: the 4 row groups of a lane column through shuffles, then the 4
    // centroid quarters through LDS; fp32: 4 quarters x 2 half-waves in LDS
    constexpr int NQ = M16 ? 4 : 8;  // candidates per point in LDS
    if constexpr (M16) {
#pragma unroll
        for (int pb = 0; pb < 8; ++pb) {
            float sc = best[pb];
            int32_t ix = bidx[pb];
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float so = __shfl_xor(sc, o);
                const int32_t io = __shfl_xor(ix, o);
                const bool take = so > sc || (so == sc && io < ix);
                sc = take ? so : sc;
                ix = take ? io : ix;
            }
            if (g == 0) {
                const int p = wp * 128 + pb * 16 + c16;
                s_best[wc * kSdP + p] = sc;
                s_idx[wc * kSdP + p] = ix;
            }
        }
    } else {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int p = wp * 128 + cb * 32 + col;
            s_best[(wc * 2 + h) * kSdP + p] = best[cb];
            s_idx[(wc * 2 + h) * kSdP + p] = bidx[cb] + 4 * h;
        }
    }
    __syncthreads();
    if (tid < kSdP) {
        const int p = tid;
        float sc = s_best[p];
        int32_t i = s_idx[p];
        for (int j = 1; j < NQ; ++j) {
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
    constexpr int EC = kSdRowB / sizeof(T);  // elements per row chunk
    // direct loads: whole chunks, full tiles, 32-bit byte offsets per problem
    const bool dma = d % EC == 0 && K >= kSdK && N * (int64_t)d * (int64_t)sizeof(T) < ((int64_t)1 << 32) &&
                     K * (int64_t)d * (int64_t)sizeof(T) < ((int64_t)1 << 32);
    // rows that are not whole slots: the widest load unit dividing the stride
    const int unit = d % (8 / (int)sizeof(T)) == 0 ? 8 : (sizeof(T) == 2 && d % 2 == 0 ? 4 : 0);
    const int smallk = K < kSdK ? 1 : 0;
    const int variant = dma            ? 4
                        : d % V == 0   ? 2 + smallk
                        : unit == 8    ? 5 + smallk
                        : unit == 4    ? 7 + smallk
                                       : smallk;
    using Kern = void (*)(const T*, const T*, const float*, int32_t*, float*, int64_t, int64_t, int);
    const Kern kerns[9] = {k_assign_splitd<T, false, false, false>, k_assign_splitd<T, false, true, false>,
                           k_assign_splitd<T, true, false, false>, k_assign_splitd<T, true, true, false>,
                           k_assign_splitd<T, true, false, true>,
                           k_assign_splitd<T, false, false, false, 8>, k_assign_splitd<T, false, true, false, 8>,
                           k_assign_splitd<T, false, false, false, 4>, k_assign_splitd<T, false, true, false, 4>};
    const Kern kern = kerns[variant];
    static LdsAttr attr[9];
    hipError_t e = ensure_lds(attr[variant], reinterpret_cast<const void*>(kern), (int)lds);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((N + kSdP - 1) / kSdP), (unsigned)B);
    hipLaunchKernelGGL(kern, grid, dim3(kSdWaves * kWave), lds, s, static_cast<const T*>(X),
                       static_cast<const T*>(C), bias, labels, min_dist, N, K, d);
    return hipGetLastError();
}

}  // namespace
}  // namespace fk
