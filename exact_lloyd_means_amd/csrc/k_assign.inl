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
//    32 rows stream HBM/L2 -> registers -> a ring of three LDS buffers, one
//    barrier per tile.
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


// Direct global -> LDS loads (gfx950 global_load_lds_dword{,x4}): lane i
// of the wave fetches base + voff and the data lands at LDS byte
// lds + 16 i (4 i for the 4-byte form); lds must be wave-uniform.  Written
// as inline assembly so the compiler does not order every later LDS access
// behind the load (it cannot tell which LDS bytes the load writes); the
// kernel waits for them itself (wait_vm).  The LDS address goes through m0,
// which is saved and restored around the load (the load reads it at issue).
// The loads write no vector register.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(lds), "s"(base)
        : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(lds), "s"(base)
        : "memory");
}
// Waits until at most N vector memory operations of this wave are in
// flight (s_waitcnt vmcnt(N); the LDS and export counters are not waited on).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

constexpr int kAssignBK = 32;    // centroids per tile (one MFMA row block)
constexpr int kAssignWaves = 8;  // two waves per SIMD, one workgroup per CU
constexpr int kAssignRing = 4;   // centroid tiles resident in LDS at once
constexpr int kLdsBytes = 160 * 1024;

// LDS of a workgroup: a ring of centroid tiles (rows padded by 16 bytes so
// the fragment reads are bank-conflict free) and their bias values.
constexpr int assign_lds(int Q) {
    return kAssignRing * (kAssignBK * (2 * Q * 16 + 16) + kAssignBK * 4);
}

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

// The same 16 bytes read in U-byte units (U = 8, 4 or sizeof(T), dividing
// the row stride d * sizeof(T)): for rows that are not whole 16-byte
// chunks, where a 16-byte load would be misaligned.  A unit lies wholly
// before or after d; units past d read as zero.
template <typename T, int U>
__device__ inline u32x4 load_chunk_units(const T* __restrict__ base, int64_t row, int64_t rows,
                                         int d, int e0) {
    constexpr int EU = U / (int)sizeof(T);  // elements per unit
    u32x4 out = {0u, 0u, 0u, 0u};
    if (row >= rows) return out;
    const T* p = base + row * (int64_t)d + e0;
    uint16_t h[8];
    uint32_t w[4];
    uint64_t q[2];
#pragma unroll
    for (int u = 0; u < 16 / U; ++u) {
        const bool in = e0 + u * EU < d;
        if constexpr (U == 8) q[u] = in ? *reinterpret_cast<const uint64_t*>(p + u * EU) : 0ull;
        if constexpr (U == 4) w[u] = in ? *reinterpret_cast<const uint32_t*>(p + u * EU) : 0u;
        if constexpr (U == 2) h[u] = in ? *reinterpret_cast<const uint16_t*>(p + u * EU) : (uint16_t)0;
    }
    if constexpr (U == 8) __builtin_memcpy(&out, q, 16);
    if constexpr (U == 4) __builtin_memcpy(&out, w, 16);
    if constexpr (U == 2) __builtin_memcpy(&out, h, 16);
    return out;
}

// Q  = 16-byte chunks per half row (HR = Q * 16 / sizeof(T) dimensions),
// NB = 32-point column blocks held by each wave,
// VEC   = d is a multiple of the 16-byte chunk (rows load as whole chunks),
// EXACT = d equals the padded row length 2*HR (no column checks at all),
// SMALLK = K < 32: the single tile is padded with -inf-bias rows.  For
//   K >= 32 the last tile instead starts at K-32 and overlaps the previous
//   one; seeing a centroid twice cannot change a strict-">" running argmax
//   (same score, later in the scan), so no padding is needed.
//
// A workgroup takes one item (8*NB*32 points of one problem) and loads the
// X fragments of its points straight into registers, where they stay for
// the whole K loop.
//
// Pipeline per wave (iteration t computes the MFMAs of tile t+1 and the
// epilogue of tile t):
//   * centroid tiles move HBM/L2 -> two register staging sets -> a ring of
//     four LDS buffers (tile j in buffer j mod 4, so with the loop unrolled
//     four times every LDS address is a constant offset): tile t+4 is loaded
//     in iteration t and stored to LDS at the end of iteration t+1;
//   * the centroid fragments and bias of tile t+2 are read from LDS during
//     iteration t, right after the MFMA that frees their registers, so the
//     reads of all waves spread over a whole tile instead of queueing behind
//     the barrier;
//   * the MFMAs of tile t+1 go out slot by slot (a slot = the NB MFMAs
//     sharing one centroid fragment and k-step) and each slot is preceded by
//     a slice of tile t's compare / select epilogue; scheduling barriers pin
//     that order, so each MFMA runs on the matrix unit while the wave's next
//     slice runs on the vector unit;
//   * one barrier per tile.
template <typename T, int Q, int NB, bool VEC, bool EXACT, bool SMALLK>
__global__ __launch_bounds__(kAssignWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_assign(const T* __restrict__ X, const T* __restrict__ C, const float* __restrict__ bias,
              int32_t* __restrict__ labels, float* __restrict__ min_dist, int64_t B, int64_t N,
              int64_t K, int d) {
    using M = Mfma<T>;
    constexpr int V = 16 / sizeof(T);
    constexpr int HR = Q * V;                          // dimensions per half row
    constexpr int RC = 2 * Q;                          // 16-byte chunks per padded row
    constexpr int ROWB = RC * 16 + 16;                 // LDS bytes per centroid row (padded)
    constexpr int TILEB = kAssignBK * ROWB;
    constexpr int CHUNKS = kAssignBK * RC;             // 16-byte chunks per centroid tile
    constexpr int NT = kAssignWaves * kWave;
    constexpr int PER = (CHUNKS + NT - 1) / NT;
    constexpr int PTS = kAssignWaves * NB * 32;        // points per item
    constexpr int kSlots = Q * M::kSteps;
    // fragments of the next tile prefetched during an iteration, and the slot
    // after which the next tile's bias is read (late, to keep it out of the
    // registers for most of the iteration)
    constexpr int P = Q <= 4 ? Q : 4;
    constexpr int kBiasSlot = kSlots > 3 ? kSlots - 3 : 0;
    static_assert(!EXACT || VEC, "EXACT implies VEC");

    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* s_tile = smem;                                                      // [ring][TILEB]
    float* s_bias = reinterpret_cast<float*>(smem + kAssignRing * TILEB);     // [ring][BK]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int col = lane & 31;
    const int K32 = (int)K;
    const int ntiles = (int)((K + kAssignBK - 1) / kAssignBK);
    const int lastbase = SMALLK ? 0 : K32 - kAssignBK;
    const int64_t nbpp = (N + PTS - 1) / PTS;          // items per problem
    const int64_t items = B * nbpp;

    // ---- centroid tile staging (registers -> LDS).  Thread tid always moves
    // the same (row, chunk) pairs of a tile, so each load is a uniform tile
    // base plus a loop-invariant per-thread offset.  Chunks past d re-read
    // the row's last chunk: the X side of those dimensions is zero, so they
    // add nothing.  Loads are issued for every t (a t past the last tile
    // re-reads the last tile) so the loop has no branches around them.
    int crow[PER], ccol[PER];
    uint32_t goff[PER];
    // A tile of fewer chunks than threads (d <= 16): each chunk is loaded
    // and stored by NT / CHUNKS threads (same value, same place), so no
    // thread waits behind a branch and the tile loop stays one block.
    static_assert(CHUNKS >= NT || NT % CHUNKS == 0, "whole copies of the tile");
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = CHUNKS < NT ? tid % CHUNKS : tid + u * NT;
        crow[u] = c / RC;
        ccol[u] = c % RC;
        const int cofs = EXACT ? ccol[u] * V : min(ccol[u] * V, d - V);
        goff[u] = (uint32_t)((crow[u] * d + cofs) * (int)sizeof(T));
    }
    auto tile_base = [&](int t) { return SMALLK ? 0 : min(t * kAssignBK, lastbase); };
    struct Staged {
        u32x4 v[PER];
        float bias;
    };

    float best[NB];
    int32_t bidx[NB];
    u32x4 xf[NB][Q];
    float xsq[NB];

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t b = item / nbpp;
        const int64_t pbase = (item - b * nbpp) * PTS + (int64_t)wave * NB * 32;
        const T* __restrict__ Cb = C + b * K * d;
        const float* __restrict__ biasb = bias + b * K;

        // ---- this item's points, resident in registers for the K loop
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int q = 0; q < Q; ++q)
                xf[nb][q] = load_chunk<T, VEC>(X + b * N * d, pbase + nb * 32 + col, N, d,
                                               h * HR + q * V);
            xsq[nb] = 0.f;
            best[nb] = -INFINITY;
            bidx[nb] = 0;
        }
        if (min_dist) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < Q; ++q) xsq[nb] += M::sumsq(xf[nb][q]);
        }

        auto gload = [&](int t, Staged& st) {
            const int tbase = tile_base(t);
            const char* base = reinterpret_cast<const char*>(Cb + (int64_t)tbase * d);
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                if (CHUNKS % NT == 0 || CHUNKS < NT || u * NT + tid < CHUNKS) {
                    if constexpr (SMALLK || !VEC) {
                        st.v[u] = load_chunk<T, VEC>(Cb, tbase + crow[u], K, d, ccol[u] * V);
                    } else {
                        st.v[u] = *reinterpret_cast<const u32x4*>(base + goff[u]);
                    }
                }
            }
            if constexpr (SMALLK) {
                const int k = tid & (kAssignBK - 1);
                const float v = biasb[min(k, K32 - 1)];
                st.bias = k < K32 ? v : -INFINITY;
            } else {
                st.bias = biasb[tbase + (tid & (kAssignBK - 1))];
            }
        };
        auto sstore = [&](int buf, const Staged& st) {
#pragma unroll
            for (int u = 0; u < PER; ++u)
                if (CHUNKS % NT == 0 || CHUNKS < NT || u * NT + tid < CHUNKS)
                    *reinterpret_cast<u32x4*>(s_tile + buf * TILEB + crow[u] * ROWB +
                                              ccol[u] * 16) = st.v[u];
            // every thread stores its bias value (identical stores per slot),
            // so the loop body has no branch
            s_bias[buf * kAssignBK + (tid & (kAssignBK - 1))] = st.bias;
        };
        // this lane's centroid fragment q of the tile in LDS buffer buf
        auto frag = [&](int buf, int q) -> u32x4 {
            return *reinterpret_cast<const u32x4*>(s_tile + buf * TILEB + col * ROWB +
                                                   (h * Q + q) * 16);
        };
        // bias of this lane's accumulator rows 8g + 4h + i (g, i = 0..3)
        auto bias_vec = [&](int buf) -> floatx16 {
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
            return bv;
        };

        // Running (max score, lowest index) over the rows of one tile's
        // scores.  Within a tile the candidate index is the lane's row offset
        // 8*(r/4) + r%4 (a small inline constant, -1 = no improvement in this
        // tile); rows ascend with r, so strict > keeps the lowest index.  The
        // tile base is added once per tile.
        float m[NB];
        int32_t rt[NB];
        auto epi_begin = [&]() {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                m[nb] = best[nb];
                rt[nb] = -1;
            }
        };
        auto epi_rows = [&](const floatx16(&sc)[NB], int r0, int r1) {
#pragma unroll
            for (int r = r0; r < r1; ++r) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float s = sc[nb][r];
                    // written as "keep" so both selects take the 2-operand form
                    const bool keep = !(s > m[nb]);
                    m[nb] = keep ? m[nb] : s;
                    rt[nb] = keep ? rt[nb] : 8 * (r >> 2) + (r & 3);
                }
            }
        };
        auto epi_end = [&](int t) {
            const int32_t kb = tile_base(t);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                best[nb] = m[nb];
                bidx[nb] = rt[nb] >= 0 ? kb + rt[nb] : bidx[nb];
            }
        };

        floatx16 acc[2][NB];
        Staged st[2];
        u32x4 a[Q];    // centroid fragments of the tile whose MFMAs run next
        floatx16 bv;   // and its bias

        // ---- prologue: tiles 0, 1, 2 into LDS, tile 3 staged; tile 0's
        // MFMAs; tile 1's first fragments and bias prefetched
        gload(0, st[0]);
        gload(1, st[1]);
        sstore(0, st[0]);
        sstore(1, st[1]);
        gload(2, st[0]);
        gload(3, st[1]);
        sstore(2, st[0]);
        __syncthreads();
        bv = bias_vec(0);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const u32x4 f = frag(0, q);
#pragma unroll
            for (int e = 0; e < M::kSteps; ++e)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[0][nb] = M::step(f, xf[nb][q], (q == 0 && e == 0) ? bv : acc[0][nb], e);
        }
#pragma unroll
        for (int q = 0; q < P; ++q) a[q] = frag(1, q);
        bv = bias_vec(1);

        // ---- iteration t (t + 1 < ntiles), i = t mod 4.  On entry
        // acc[t mod 2] holds tile t's scores, a[0..P) and bv tile t+1's first
        // fragments and bias; LDS holds tiles t+1 and t+2; staging set
        // (t+1) mod 2 holds tile t+3.
        auto iteration = [&](int t, int i) {
            floatx16(&cur)[NB] = acc[(i & 1) ^ 1];
            const floatx16(&prv)[NB] = acc[i & 1];
            const int b1 = (i + 1) % kAssignRing;  // tile t+1
            const int b2 = (i + 2) % kAssignRing;  // tile t+2
            const int b3 = (i + 3) % kAssignRing;  // receives tile t+3
            gload(t + 4, st[i & 1]);
            u32x4 nx[P];
            floatx16 nbv;
            __builtin_amdgcn_sched_barrier(0);
            epi_begin();
#pragma unroll
            for (int sl = 0; sl < kSlots; ++sl) {
                const int q = sl / M::kSteps;
                const int e = sl % M::kSteps;
                epi_rows(prv, 16 * sl / kSlots, 16 * (sl + 1) / kSlots);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    cur[nb] = M::step(a[q], xf[nb][q], sl == 0 ? bv : cur[nb], e);
                if (e == M::kSteps - 1) {
                    // a[q] is free: read the fragment needed P slots later
                    const int v = q + P;
                    if (v < Q)
                        a[v] = frag(b1, v);
                    else
                        nx[v - Q] = frag(b2, v - Q);
                }
                if (sl == kBiasSlot) nbv = bias_vec(b2);
                __builtin_amdgcn_sched_barrier(0);
            }
            epi_end(t);
#pragma unroll
            for (int q = 0; q < P; ++q) a[q] = nx[q];
            bv = nbv;
            sstore(b3, st[(i & 1) ^ 1]);
            __syncthreads();
        };
        auto final_epilogue = [&](int t, const floatx16(&sc)[NB]) {
            epi_begin();
            epi_rows(sc, 0, 16);
            epi_end(t);
        };
        int t = 0;
        for (; t + 4 < ntiles; t += 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) iteration(t + i, i);
        }
        // the last one to four tiles
        switch (ntiles - t) {
            case 1:
                final_epilogue(t, acc[0]);
                break;
            case 2:
                iteration(t, 0);
                final_epilogue(t + 1, acc[1]);
                break;
            case 3:
                iteration(t, 0);
                iteration(t + 1, 1);
                final_epilogue(t + 2, acc[0]);
                break;
            default:
                iteration(t, 0);
                iteration(t + 1, 1);
                iteration(t + 2, 2);
                final_epilogue(t + 3, acc[1]);
                break;
        }

        // ---- merge the two half-waves that hold the same point; write labels
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float sc = best[nb];
            int32_t i = bidx[nb] + 4 * h;
            const float so = __shfl_xor(sc, 32);
            const int32_t io = __shfl_xor(i, 32);
            if (so > sc || (so == sc && io < i)) {
                sc = so;
                i = io;
            }
            const float xx = xsq[nb] + __shfl_xor(xsq[nb], 32);
            const int64_t j = pbase + nb * 32 + col;
            if (h == 0 && j < N) {
                labels[b * N + j] = i;
                if (min_dist) min_dist[b * N + j] = xx - 2.f * sc;
            }
        }
        __syncthreads();  // the next item's prologue rewrites the ring
    }
}


template <typename T, int Q, int NB, bool VEC, bool EXACT, bool SMALLK>
hipError_t launch_assign_t(const void* X, const void* C, const float* bias, int32_t* labels,
                           float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                           hipStream_t s) {
    constexpr int lds = assign_lds(Q);
    static_assert(lds <= kLdsBytes, "LDS budget");
    constexpr int PTS = kAssignWaves * NB * 32;
    auto kern = k_assign<T, Q, NB, VEC, EXACT, SMALLK>;
    static LdsAttr attr;
    hipError_t e = ensure_lds(attr, reinterpret_cast<const void*>(kern), lds);
    if (e != hipSuccess) return e;
    // one workgroup per item
    const int64_t grid = B * ((N + PTS - 1) / PTS);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kAssignWaves * kWave), lds, s,
                       static_cast<const T*>(X), static_cast<const T*>(C), bias, labels, min_dist,
                       B, N, K, d);
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
    if (need <= QQ) {                                                                         \
        if (K < kAssignBK)                                                                    \
            return vec ? launch_assign_t<T, QQ, NBB, true, false, true>(X, C, bias, labels,     \
                                                                        min_dist, B, N, K, d, s) \
                       : launch_assign_t<T, QQ, NBB, false, false, true>(X, C, bias, labels,    \
                                                                         min_dist, B, N, K, d, s); \
        if (vec && d == 2 * QQ * V)                                                           \
            return launch_assign_t<T, QQ, NBB, true, true, false>(X, C, bias, labels, min_dist, \
                                                                  B, N, K, d, s);             \
        if (vec)                                                                              \
            return launch_assign_t<T, QQ, NBB, true, false, false>(X, C, bias, labels, min_dist, \
                                                                   B, N, K, d, s);            \
        return launch_assign_t<T, QQ, NBB, false, false, false>(X, C, bias, labels, min_dist, B, \
                                                                N, K, d, s);                  \
    }
    FK_ASSIGN_CASE(1, 2)
    FK_ASSIGN_CASE(2, 2)
    FK_ASSIGN_CASE(4, 2)
    FK_ASSIGN_CASE(8, 2)
    FK_ASSIGN_CASE(16, 1)
#undef FK_ASSIGN_CASE
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace fk
