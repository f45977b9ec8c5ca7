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

constexpr int kAssignBK = 32;  // centroids per tile (one MFMA row block)
constexpr int kAssignWaves = 8;  // two waves per SIMD, one workgroup per CU
constexpr int kLdsBytes = 160 * 1024;

// LDS of a workgroup: optionally the X block of the next item (points x
// padded row), two centroid tiles (rows padded by 16 bytes) and their bias.
constexpr int assign_lds(int Q, int NB, bool prefx) {
    return (prefx ? kAssignWaves * NB * 32 * 2 * Q * 16 : 0) + 2 * kAssignBK * (2 * Q * 16 + 16) +
           2 * kAssignBK * 4;
}
// Prefetching the next item's X block through LDS (persistent workgroups)
// measured no faster on MI355X than loading X at the item start, so it is
// off; the path stays for experiments with other shapes.
constexpr bool assign_prefetch_x(int Q, int NB) {
    return false && assign_lds(Q, NB, true) <= kLdsBytes;
}
// Staging register sets for centroid tiles: four (loads two iterations
// ahead of their LDS store) when a thread moves at most two chunks per
// tile, else two (one iteration ahead).
constexpr int assign_sets(int Q) {
    return (kAssignBK * 2 * Q + kAssignWaves * kWave - 1) / (kAssignWaves * kWave) <= 2 ? 4 : 2;
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

// Q  = 16-byte chunks per half row (HR = Q * 16 / sizeof(T) dimensions),
// NB = 32-point column blocks held by each wave,
// VEC   = d is a multiple of the 16-byte chunk (rows load as whole chunks),
// EXACT = d equals the padded row length 2*HR (no column checks at all),
// SMALLK = K < 32: the single tile is padded with -inf-bias rows.  For
//   K >= 32 the last tile instead starts at K-32 and overlaps the previous
//   one; seeing a centroid twice cannot change a strict-">" running argmax
//   (same score, later in the scan), so no padding is needed.
//
// An item is a block of 8*NB*32 points of one problem.  With PREFX the
// kernel is persistent (one workgroup per CU walks the items) and, while it
// runs the K loop of an item, prefetches the X block of its next item into
// LDS, one 16-byte chunk per thread per tile iteration; the block is copied
// into registers at the item switch, so no wave waits for X from memory.
// Without PREFX (rows too long for the LDS budget) each workgroup takes one
// item and loads its X straight into registers.
//
// Pipeline per wave and item: the MFMAs of tile t+1 are issued interleaved
// with the compare / select epilogue of tile t (sched_group_barrier); the
// centroid tiles reach LDS through NSET staging register sets, loaded D
// tiles ahead of use; one barrier per tile.
template <typename T, int Q, int NB, bool VEC, bool EXACT, bool SMALLK>
__global__ __launch_bounds__(kAssignWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_assign(const T* __restrict__ X, const T* __restrict__ C, const float* __restrict__ bias,
              int32_t* __restrict__ labels, float* __restrict__ min_dist, int64_t B, int64_t N,
              int64_t K, int d) {
    using M = Mfma<T>;
    constexpr bool PREFX = assign_prefetch_x(Q, NB);
    constexpr int NSET = assign_sets(Q);
    constexpr int D = NSET == 2 ? 3 : 4;               // load tile t+D in iteration t
    constexpr int V = 16 / sizeof(T);
    constexpr int HR = Q * V;                          // dimensions per half row
    constexpr int RC = 2 * Q;                          // 16-byte chunks per padded row
    constexpr int ROWB = RC * 16 + 16;                 // LDS bytes per centroid row (padded)
    constexpr int TILEB = kAssignBK * ROWB;
    constexpr int CHUNKS = kAssignBK * RC;             // 16-byte chunks per centroid tile
    constexpr int NT = kAssignWaves * kWave;
    constexpr int PER = (CHUNKS + NT - 1) / NT;
    constexpr int PTS = kAssignWaves * NB * 32;        // points per item
    constexpr int XPT = PTS * RC / NT;                 // X chunks per thread per item
    constexpr int XB = PREFX ? PTS * RC * 16 : 0;      // LDS bytes of the X buffer
    static_assert(!EXACT || VEC, "EXACT implies VEC");
    static_assert((PTS * RC) % NT == 0, "X chunks divide evenly");
    static_assert(D != 2 + NSET && (D - 2) % NSET != 0, "load and store sets differ");

    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* s_x = smem;                                               // [PTS][RC] swizzled
    char* s_tile = smem + XB;                                       // [2][TILEB]
    float* s_bias = reinterpret_cast<float*>(s_tile + 2 * TILEB);   // [2][BK]

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

    // ---- X block staging: chunk c of thread tid is point p, logical chunk
    // lc of that point; LDS slot p*RC + (lc ^ (p % RC)) (conflict-free reads)
    const int N32 = (int)N;
    // chunk c of this thread for the item whose X rows start at Xi and whose
    // first point is row r0 of its problem
    auto x_load = [&](const T* Xi, int r0, int c) -> u32x4 {
        const int g = c * NT + tid;
        const int p = g / RC;
        const int lc = g % RC;
        const int row = min(r0 + p, N32 - 1);  // rows past N: any finite data
        if constexpr (VEC) {
            const int e0 = EXACT ? lc * V : min(lc * V, d - V);  // zeroed after the copy
            return *reinterpret_cast<const u32x4*>(Xi + (int64_t)row * d + e0);
        } else {
            return load_chunk<T, false>(Xi, row, N, d, lc * V);
        }
    };
    auto x_store = [&](int c, u32x4 v) {
        const int g = c * NT + tid;
        const int p = g / RC;
        const int lc = g % RC;
        *reinterpret_cast<u32x4*>(s_x + (p * RC + (lc ^ (p & (RC - 1)))) * 16) = v;
    };

    // ---- centroid tile staging (registers -> LDS).  Thread tid always moves
    // the same (row, chunk) pairs of a tile, so each load is a uniform tile
    // base plus a loop-invariant per-thread offset.  Chunks past d re-read
    // the row's last chunk: the X side of those dimensions is zero, so they
    // add nothing.  Loads are issued for every t (a t past the last tile
    // re-reads the last tile) so the loop has no branches around them.
    int crow[PER], ccol[PER];
    uint32_t goff[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = tid + u * NT;
        crow[u] = c / RC;
        ccol[u] = c % RC;
        const int cofs = EXACT ? ccol[u] * V : min(ccol[u] * V, d - V);
        goff[u] = (uint32_t)((crow[u] * d + cofs) * (int)sizeof(T));
    }
    auto tile_base = [&](int t) { return SMALLK ? 0 : min(t * kAssignBK, lastbase); };
    struct Staged {
        u32x4 v[PER];
        float bias;
        u32x4 x;  // one chunk of the next item's X block (PREFX)
    };

    float best[NB];
    int32_t bidx[NB];
    u32x4 xf[NB][Q];
    float xsq[NB];

    int64_t item = blockIdx.x;
    if (item >= items) return;
    if constexpr (PREFX) {  // first item: its X block straight into LDS
        const int64_t b0 = item / nbpp;
        const T* Xi = X + b0 * N * d;
        const int r0 = (int)(item - b0 * nbpp) * PTS;
        for (int c = 0; c < XPT; ++c) x_store(c, x_load(Xi, r0, c));
        __syncthreads();
    }

    for (; item < items; item += gridDim.x) {
        const int64_t next = PREFX && item + gridDim.x < items ? item + gridDim.x : item;
        const int64_t bn = next / nbpp;
        const T* Xn = X + bn * N * d;                  // next item's problem
        const int rn = (int)(next - bn * nbpp) * PTS;  // next item's first point
        const int64_t b = item / nbpp;
        const int64_t pbase = (item - b * nbpp) * PTS + (int64_t)wave * NB * 32;
        const T* __restrict__ Cb = C + b * K * d;
        const float* __restrict__ biasb = bias + b * K;

        // ---- this item's points, resident in registers for the K loop
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int p = wave * NB * 32 + nb * 32 + col;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                u32x4 v;
                if constexpr (PREFX) {
                    const int lc = h * Q + q;
                    v = *reinterpret_cast<const u32x4*>(s_x + (p * RC + (lc ^ (p & (RC - 1)))) * 16);
                    if (!EXACT && h * HR + q * V >= d) v = (u32x4){0u, 0u, 0u, 0u};
                } else {
                    v = load_chunk<T, VEC>(X + b * N * d, pbase + nb * 32 + col, N, d,
                                           h * HR + q * V);
                }
                xf[nb][q] = v;
            }
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
        if constexpr (PREFX) __syncthreads();  // the X buffer may now receive the next item

        auto gload = [&](int t, Staged& st) {
            const int tbase = tile_base(t);
            const char* base = reinterpret_cast<const char*>(Cb + (int64_t)tbase * d);
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                if (CHUNKS % NT == 0 || u * NT + tid < CHUNKS) {
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
            // X chunk t-D of the next item rides along with tile t (chunks
            // before 0 and past XPT-1 repeat the first / last one)
            if constexpr (PREFX) st.x = x_load(Xn, rn, min(max(t - D, 0), XPT - 1));
        };
        auto sstore = [&](int buf, const Staged& st, int t) {
#pragma unroll
            for (int u = 0; u < PER; ++u)
                if (CHUNKS % NT == 0 || u * NT + tid < CHUNKS)
                    *reinterpret_cast<u32x4*>(s_tile + buf * TILEB + crow[u] * ROWB +
                                              ccol[u] * 16) = st.v[u];
            // every thread stores its bias value (identical stores per slot),
            // so the loop body has no branch
            s_bias[buf * kAssignBK + (tid & (kAssignBK - 1))] = st.bias;
            if constexpr (PREFX) x_store(min(max(t - D, 0), XPT - 1), st.x);
        };

        // MFMAs of the tile in LDS buffer `buf`; the accumulators start at
        // the bias of their rows (8g + 4h + i, g, i = 0..3).
        auto mma = [&](int buf, floatx16 (&acc)[NB]) {
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
        };

        // Running (max score, lowest index).  Within a tile the candidate
        // index is the lane's row offset 8*(r/4) + r%4 (a small inline
        // constant, -1 = no improvement in this tile); rows ascend with r, so
        // strict > keeps the lowest index.  The tile base is added once per
        // tile.  The NB chains are independent; interleaving them spaces each
        // compare from the select that consumes it.
        auto epilogue = [&](const floatx16 (&acc)[NB], int t) {
            const int32_t kb = tile_base(t);
            float m[NB];
            int32_t rt[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                m[nb] = best[nb];
                rt[nb] = -1;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const float s = acc[nb][r];
                    // written as "keep" so both selects take the 2-operand form
                    const bool keep = !(s > m[nb]);
                    m[nb] = keep ? m[nb] : s;
                    rt[nb] = keep ? rt[nb] : 8 * (r >> 2) + (r & 3);
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                best[nb] = m[nb];
                bidx[nb] = rt[nb] >= 0 ? kb + rt[nb] : bidx[nb];
            }
        };

        floatx16 acc[2][NB];
        Staged st[NSET];
        constexpr int U = NSET == 4 ? 4 : 2;  // unroll: acc parity and set rotation repeat
        // set holding tile j: st[j % NSET]; with two sets tile 2 reuses tile
        // 0's set once tile 0 is in LDS
#pragma unroll
        for (int j = 0; j < (D < NSET ? D : NSET); ++j) gload(j, st[j]);
        sstore(0, st[0], 0);
#pragma unroll
        for (int j = NSET; j < D; ++j) gload(j, st[j % NSET]);
        __syncthreads();
        mma(0, acc[0]);
        sstore(1, st[1 % NSET], 1);
        __syncthreads();

        // iteration t (t + 1 < ntiles): tile t's scores are in acc[t&1],
        // tile t+1 is in LDS buffer (t+1)&1, tile t+2 waits in its set and
        // tile t+D is loaded.  The body is one basic block; the schedule
        // interleaves every MFMA of tile t+1 with a few epilogue instructions
        // of tile t, so the vector unit works while the matrix unit runs.
        auto iteration = [&](int t, int i) {
            gload(t + D, st[(i + D) % NSET]);
            mma((i + 1) & 1, acc[(i + 1) & 1]);
            epilogue(acc[i & 1], t);
            sstore(i & 1, st[(i + 2) % NSET], t + 2);
            constexpr int kMfma = NB * Q * M::kSteps;
            constexpr int kValuPer = (NB * 48 + kMfma - 1) / kMfma + 1;
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);                       // bias + A reads
            __builtin_amdgcn_sched_group_barrier(0x020, PER + 1 + (PREFX ? 1 : 0), 0);  // loads
#pragma unroll
            for (int k = 0; k < kMfma; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // epilogue VALU
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // next A read
            }
            __syncthreads();
        };
        int t = 0;
        for (; t + U < ntiles; t += U) {
#pragma unroll
            for (int i = 0; i < U; ++i) iteration(t + i, i);
        }
        // the last 1..U tiles: one fewer iteration, then the final epilogue
        switch (ntiles - t) {
            case 1:
                epilogue(acc[0], t);
                break;
            case 2:
                iteration(t, 0);
                epilogue(acc[1], t + 1);
                break;
            case 3:
                if constexpr (U >= 4) {
                    iteration(t, 0);
                    iteration(t + 1, 1);
                    epilogue(acc[0], t + 2);
                }
                break;
            default:
                if constexpr (U >= 4) {
                    iteration(t, 0);
                    iteration(t + 1, 1);
                    iteration(t + 2, 2);
                    epilogue(acc[1], t + 3);
                }
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

        if constexpr (PREFX) {
            // ---- complete the next item's X block.  Tile j carries X chunk
            // j-D.  Iterations 0 .. ntiles-2 loaded tiles up to ntiles-2+D
            // and stored tiles up to ntiles, so the chunks of tiles ntiles+1
            // .. ntiles+D-2 still sit in their sets and chunks from ntiles-1
            // on were never loaded.
#pragma unroll
            for (int j = 1; j <= D - 2; ++j) {
                const int tj = ntiles + j;      // tile whose set holds the chunk
                const int c = tj - D;
                if (c >= 0 && c < XPT) {
                    const int si = tj % NSET;
                    u32x4 v = st[0].x;
#pragma unroll
                    for (int k = 1; k < NSET; ++k)
                        if (si == k) v = st[k].x;
                    x_store(c, v);
                }
            }
            for (int c = max(ntiles - 1, 0); c < XPT; ++c) x_store(c, x_load(Xn, rn, c));
            __syncthreads();
        }
    }
}

template <typename T, int Q, int NB, bool VEC, bool EXACT, bool SMALLK>
hipError_t launch_assign_t(const void* X, const void* C, const float* bias, int32_t* labels,
                           float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                           hipStream_t s) {
    constexpr bool prefx = assign_prefetch_x(Q, NB);
    constexpr int lds = assign_lds(Q, NB, prefx);
    static_assert(lds <= kLdsBytes, "LDS budget");
    constexpr int PTS = kAssignWaves * NB * 32;
    auto kern = k_assign<T, Q, NB, VEC, EXACT, SMALLK>;
    static bool attr_set = false;  // one attribute call per instantiation and process
    static int cus = 0;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t items = B * ((N + PTS - 1) / PTS);
    // persistent: one workgroup per CU; otherwise one workgroup per item
    const int64_t grid = prefx ? (items < cus ? items : cus) : items;
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
    FK_ASSIGN_CASE(32, 1)
#undef FK_ASSIGN_CASE
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace fk
