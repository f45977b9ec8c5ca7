// k_assign16.inl -- fused distance + running argmin for 16-bit inputs on
// the 16x16x32 matrix instructions.
//
// Same method and pipeline as k_assign.inl (papernotes.org notes
// "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", 关键设计 1: never
// store the N x K distance matrix, keep a running (min, argmin) per point),
// with v_mfma_f32_16x16x32_{f16,bf16} in place of the 32x32x16 form.  Under
// full load the MI355X matrix units are power-limited; with random operands
// the 16x16x32 form (a quarter of the accumulator registers per instruction)
// sustains markedly more flops than the 32x32x16 form, so it is used for the
// 16-bit types.
//
// Lane layout of v_mfma_f32_16x16x32: lane l supplies A[l%16][8*(l/16) + j]
// and B[8*(l/16) + j][l%16] (j = 0..7) and holds D[4*(l/16) + i][l%16]
// (i = 0..3).  Rows are centroids, columns points: each point's 16 scores of
// a 16-centroid block are spread over the four lanes l%16 + 16*g, four each,
// and the four lanes merge once at the end.
#pragma once

#include "k_assign.inl"

namespace fk {
namespace {

// Calls f(std::integral_constant<int, I>) for I = B .. E-1: loop bodies whose
// bounds depend on an outer index stay compile-time constants.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <typename T>
struct Mfma16;

template <>
struct Mfma16<_Float16> {
    __device__ static inline floatx4 step(u32x4 a, u32x4 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                      __builtin_bit_cast(half8, b), c, 0, 0, 0);
    }
};

template <>
struct Mfma16<__bf16> {
    __device__ static inline floatx4 step(u32x4 a, u32x4 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

// LDS slot (16-byte unit within the row) of chunk ch of centroid row `row`
// in a tile whose rows hold RC chunks.  gfx950's LDS has 64 four-byte banks
// (256 bytes); a row of RC chunks covers RC of the 16 bank groups, so 16 / RC
// consecutive rows share a 256-byte bank line.  The chunk index is XORed
// with a function of the row that makes any 16 consecutive rows read at one
// chunk index land in 16 different bank groups: the fragment reads (16 rows,
// one chunk) and the staging stores (consecutive chunks) are then free of
// bank conflicts.  (Rows padded by 16 bytes instead measured four conflict
// cycles per fragment read.)
template <int RC>
__device__ __forceinline__ int lds_slot(int row, int ch) {
    constexpr int G = RC >= 16 ? 1 : 16 / RC;  // rows per 256-byte bank line
    constexpr int M = RC >= 16 ? 15 : RC - 1;
    return ch ^ ((row / G) & M);
}

// S = k-steps of 32 dimensions (d <= 32 S), NP = 16-point column blocks held
// by each wave, VEC / EXACT / SMALLK as in k_assign.  MAT: instead of the
// running argmax, every score is written to D [B][N][K] fp32 (the distance
// matrix the fused kernel exists to avoid; a baseline for comparison).
//
// Tile of 32 centroids = 2 row blocks of 16.  A slot is the NP MFMAs that
// share one centroid fragment (row block rb, k-step s), slot order s-major;
// in each slot every MFMA is followed by the epilogue of one row of tile t
// for its point block (rows spread evenly over the slots).  The ring of
// four LDS buffers, the prefetch of the next tile's fragments and bias, and
// the branch-free overlapping last tile are those of k_assign; the tiles
// reach the ring by direct global-to-LDS loads when every thread moves whole
// 16-byte chunks (DMA below), else through registers as in k_assign.
template <typename T, int S, int NP, bool VEC, bool EXACT, bool SMALLK, bool MAT, int W, int U = 2>
__device__ __forceinline__ void assign16_body(const T* __restrict__ X, const T* __restrict__ C,
                                              const float* __restrict__ bias,
                                              int32_t* __restrict__ labels,
                                              float* __restrict__ min_dist, int64_t B, int64_t N,
                                              int64_t K, int d, float* __restrict__ D) {
    using M = Mfma16<T>;
    using MS = Mfma<T>;
    constexpr int V = 8;                               // elements per 16-byte chunk
    constexpr int RC = 4 * S;                          // 16-byte chunks per row
    constexpr int ROWB = RC * 16;                      // LDS bytes per centroid row
    constexpr int TILEB = kAssignBK * ROWB;
    constexpr int CHUNKS = kAssignBK * RC;             // 16-byte chunks per centroid tile
    constexpr int NT = W * kWave;
    constexpr int PER = (CHUNKS + NT - 1) / NT;
    // Centroid tiles move global -> LDS by direct loads (no registers, no
    // LDS store instructions) when the tile is whole 16-byte chunks that
    // the waves cover evenly; otherwise through registers.
    constexpr bool DMA = VEC && !SMALLK && CHUNKS % NT == 0;
    constexpr int BIASB = DMA ? W * kWave * 4 : kAssignBK * 4;  // bias bytes per ring buffer
    constexpr int PTS = W * NP * 16;                   // points per item
    constexpr int RB = 2;                              // row blocks per tile
    constexpr int kSlots = S * RB;
    constexpr int P = kSlots <= 2 ? kSlots : 2;        // fragments prefetched for the next tile
    constexpr int kBiasSlot = kSlots > 3 ? kSlots - 3 : 0;
    constexpr int kEpiSteps = 12 * NP;                 // epilogue steps per tile (epi_op)
    static_assert(!EXACT || VEC, "EXACT implies VEC");
    // Rows that are not whole 16-byte chunks (!VEC) load in U-byte units,
    // the widest dividing the row stride (8 or 4 bytes; U = 2: element by
    // element); centroid units past d are read at the row's last unit
    // instead (the points are zero there, so any finite value does).
    constexpr bool UNITS = !VEC && !SMALLK && U >= 4;
    constexpr int NU = 16 / U, EU = U / (int)sizeof(T);  // units per chunk, elements per unit

    extern __shared__ __attribute__((aligned(16))) char smem[];
    char* s_tile = smem;                                                      // [ring][TILEB]
    float* s_bias = reinterpret_cast<float*>(smem + kAssignRing * TILEB);     // [ring][BIASB]
    const uint32_t lds_tile = (uint32_t)(uintptr_t)s_tile;
    const uint32_t lds_bias = (uint32_t)(uintptr_t)s_bias;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;     // k group of the fragments, row group of the scores
    const int col = lane & 15;
    const int K32 = (int)K;
    const int ntiles = (int)((K + kAssignBK - 1) / kAssignBK);
    const int lastbase = SMALLK ? 0 : K32 - kAssignBK;
    const int64_t nbpp = (N + PTS - 1) / PTS;
    const int64_t items = B * nbpp;

    int crow[PER], ccol[PER];
    uint32_t goff[PER], soff[PER];
    // A tile of fewer chunks than threads (d <= 32): each chunk is loaded
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
        soff[u] = (uint32_t)(crow[u] * ROWB + lds_slot<RC>(crow[u], ccol[u]) * 16);
        if constexpr (DMA) {
            // direct load u of this wave fills LDS chunks (u W + wave) 64 + lane
            // of the tile in order; the chunk that belongs there (the slot
            // map is its own inverse) is the one this lane fetches
            const int pos = (u * W + wave) * kWave + lane;
            const int row = pos / RC, ch = lds_slot<RC>(row, pos % RC);
            const int eofs = EXACT ? ch * V : min(ch * V, d - V);
            goff[u] = (uint32_t)((row * d + eofs) * (int)sizeof(T));
        }
    }
    // UNITS: byte offsets (within a tile) of the units of this thread's chunks
    uint32_t uoff[UNITS ? PER : 1][UNITS ? NU : 1];
    if constexpr (UNITS) {
#pragma unroll
        for (int u = 0; u < PER; ++u)
#pragma unroll
            for (int h = 0; h < NU; ++h)
                uoff[u][h] = (uint32_t)((crow[u] * d + min(ccol[u] * V + h * EU, d - EU)) *
                                        (int)sizeof(T));
    }
    // LDS byte offset (within a tile, row block 0) of the fragment of k-step
    // s this lane reads: row col, chunk 4 s + g, one register per k-step
    uint32_t faddr[S];
#pragma unroll
    for (int s = 0; s < S; ++s)
        faddr[s] = (uint32_t)(col * ROWB + lds_slot<RC>(col, 4 * s + g) * 16);
    auto tile_base = [&](int t) { return SMALLK ? 0 : min(t * kAssignBK, lastbase); };
    struct Staged {
        u32x4 v[PER];
        float bias;
    };

    float best[NP];
    int32_t bidx[NP];
    u32x4 xf[NP][S];

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t b = item / nbpp;
        const int64_t pbase = (item - b * nbpp) * PTS + (int64_t)wave * NP * 16;
        const T* __restrict__ Cb = C + b * K * d;
        const float* __restrict__ biasb = bias + b * K;

        // ---- this item's points, resident in registers for the K loop:
        // k-step s of point column col holds dimensions 32 s + 8 g .. + 7
#pragma unroll
        for (int np = 0; np < NP; ++np) {
#pragma unroll
            for (int s = 0; s < S; ++s)
                xf[np][s] = UNITS ? load_chunk_units<T, UNITS ? U : 8>(
                                        X + b * N * d, pbase + np * 16 + col, N, d, 32 * s + 8 * g)
                                  : load_chunk<T, VEC>(X + b * N * d, pbase + np * 16 + col, N, d,
                                                       32 * s + 8 * g);
            best[np] = -INFINITY;
            bidx[np] = 0;
        }

        auto gload = [&](int t, Staged& st) {
            const int tbase = tile_base(t);
            const char* base = reinterpret_cast<const char*>(Cb + (int64_t)tbase * d);
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                if (CHUNKS % NT == 0 || CHUNKS < NT || u * NT + tid < CHUNKS) {
                    if constexpr (UNITS) {
                        uint64_t q[2];
                        uint32_t w[4];
#pragma unroll
                        for (int h = 0; h < NU; ++h) {
                            if constexpr (U == 8)
                                q[h] = *reinterpret_cast<const uint64_t*>(base + uoff[u][h]);
                            else
                                w[h] = *reinterpret_cast<const uint32_t*>(base + uoff[u][h]);
                        }
                        if constexpr (U == 8)
                            __builtin_memcpy(&st.v[u], q, 16);
                        else
                            __builtin_memcpy(&st.v[u], w, 16);
                    } else if constexpr (SMALLK || !VEC) {
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
                    *reinterpret_cast<u32x4*>(s_tile + buf * TILEB + soff[u]) = st.v[u];
            s_bias[buf * kAssignBK + (tid & (kAssignBK - 1))] = st.bias;
        };
        // Direct loads of tile t into LDS buffer buf: PER 16-byte loads per
        // lane for the rows, one 4-byte load per lane for the bias (each
        // wave fills its own copy of the 32 values, twice).
        auto dma_tile = [&](int t, int buf) {
            const uint32_t tb = (uint32_t)tile_base(t);
            const uint32_t rows = tb * (uint32_t)d * (uint32_t)sizeof(T);
#pragma unroll
            for (int u = 0; u < PER; ++u)
                lds_dma16(Cb, rows + goff[u],
                          __builtin_amdgcn_readfirstlane(lds_tile + buf * TILEB + (u * W + wave) * 1024));
            lds_dma4(biasb, (tb + (lane & (kAssignBK - 1))) * 4u,
                     __builtin_amdgcn_readfirstlane(lds_bias + buf * BIASB + wave * kWave * 4));
        };
        // fragment of slot sl (k-step sl / RB, row block sl % RB) of the tile
        // in LDS buffer buf: row 16 rb + col, chunk 4 s + g (at its slot)
        auto frag = [&](int buf, int sl) -> u32x4 {
            const int s = sl / RB, rb = sl % RB;
            return *reinterpret_cast<const u32x4*>(s_tile + buf * TILEB + rb * 16 * ROWB +
                                                   faddr[s]);
        };
        // bias of this lane's accumulator rows 16 rb + 4 g + i
        auto bias_vec = [&](int buf, floatx4 (&bv)[RB]) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                bv[rb] = *reinterpret_cast<const floatx4*>(
                    s_bias + buf * (BIASB / 4) + (DMA ? wave * kWave : 0) + 16 * rb + 4 * g);
        };

        // MAT: lane (g, col) holds scores of centroids 16 rb + 4 g + i
        // (i = 0..3) of point col of each block
        auto mat_store = [&](int t, const floatx4(&sc)[RB][NP]) {
            const int32_t kb = tile_base(t);
#pragma unroll
            for (int np = 0; np < NP; ++np) {
                const int64_t j = pbase + np * 16 + col;
                if (j >= N) continue;
                float* row = D + (b * N + j) * K;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const int k0 = kb + 16 * rb + 4 * g;
                    if (!SMALLK && (K32 & 3) == 0) {  // then kb, k0 and each row are 16-byte aligned
                        *reinterpret_cast<floatx4*>(row + k0) = sc[rb][np];
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (k0 + i < K32) row[k0 + i] = sc[rb][np][i];
                    }
                }
            }
        };
        // Running (max score, lowest index) per point block.  A tile gives
        // each lane 8 rows of each point block, centroid 16 rb + 4 g + i
        // of the tile for row r = 4 rb + i; rows ascend with the index, so
        // the decision is that of a strict > over ascending rows against
        // the running best.  It is taken in few vector operations: the tile
        // maximum (with the running best) by a tree of three-input maxima,
        // the lowest row holding it by a descending chain of
        // compare-and-selects, then one update.  The maximum of finite and
        // infinite scores is one of them, NaN scores are passed over by the
        // maxima and equal nothing, and best never becomes NaN, so the row
        // found is the first whose score exceeds everything before it (a
        // -0/+0 tie may leave best with the other sign of zero, which
        // compares equal).  Twelve steps per point block, one block
        // after the other, so each block's scores die early: 4 maxima, 7
        // chain links, 1 update.
        static_assert(RB == 2, "8 rows per lane and tile");
        float h0, h1, h2, tm;
        int32_t ti;
        auto epi_op = [&](const floatx4(&sc)[RB][NP], int op, int32_t kb) {
            const int np = op / 12, j = op % 12;
            auto sv = [&](int r) { return sc[r >> 2][np][r & 3]; };
            if (j == 0) {
                h0 = fmaxf(fmaxf(sv(0), sv(1)), sv(2));
            } else if (j == 1) {
                h1 = fmaxf(fmaxf(sv(3), sv(4)), sv(5));
            } else if (j == 2) {
                h2 = fmaxf(fmaxf(sv(6), sv(7)), best[np]);
            } else if (j == 3) {
                tm = fmaxf(fmaxf(h0, h1), h2);
            } else if (j < 11) {
                const int r = 10 - j;  // rows 6 .. 0
                const int32_t keep = r == 6 ? 16 + 3 : ti;
                ti = sv(r) == tm ? 16 * (r >> 2) + (r & 3) : keep;
            } else {
                const bool up = tm > best[np];
                best[np] = tm;
                bidx[np] = up ? kb + ti : bidx[np];
            }
        };

        floatx4 acc[2][RB][NP];
        Staged st[DMA ? 1 : 2];
        u32x4 a[kSlots];  // centroid fragments of the tile whose MFMAs run next
        floatx4 bv[RB];   // and its bias

        // ---- prologue: tiles 0, 1, 2 into LDS (and tile 3 on its way);
        // tile 0's MFMAs; tile 1's first fragments and bias prefetched
        if constexpr (DMA) {
#pragma unroll
            for (int q = 0; q < kAssignRing; ++q) dma_tile(q, q);
            wait_vm<PER + 1>();  // tiles 0..2 have landed
        } else {
            gload(0, st[0]);
            gload(1, st[1]);
            sstore(0, st[0]);
            sstore(1, st[1]);
            gload(2, st[0]);
            gload(3, st[1]);
            sstore(2, st[0]);
        }
        __syncthreads();
        bias_vec(0, bv);
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) {
            const u32x4 f = frag(0, sl);
            const int s = sl / RB, rb = sl % RB;
#pragma unroll
            for (int np = 0; np < NP; ++np)
                acc[0][rb][np] = M::step(f, xf[np][s], s == 0 ? bv[rb] : acc[0][rb][np]);
        }
#pragma unroll
        for (int q = 0; q < P; ++q) a[q] = frag(1, q);
        bias_vec(1, bv);
        // iteration 0 reloads buffer 0 (DMA); the register path stores tile 3
        // into buffer 3 at its end
        if constexpr (DMA) __syncthreads();

        // ---- iteration t (t + 1 < ntiles), i = t mod 4 (see k_assign)
        auto iteration = [&](int t, int i) {
            floatx4(&cur)[RB][NP] = acc[(i & 1) ^ 1];
            const floatx4(&prv)[RB][NP] = acc[i & 1];
            const int b1 = (i + 1) % kAssignRing;  // tile t+1
            const int b2 = (i + 2) % kAssignRing;  // tile t+2
            const int b3 = (i + 3) % kAssignRing;  // receives tile t+3
            // tile t + 4 replaces tile t (read for the last time before the
            // previous barrier); it is first read two iterations later
            if constexpr (DMA)
                dma_tile(t + 4, i);
            else
                gload(t + 4, st[i & 1]);
            u32x4 nx[P];
            floatx4 nbv[RB];
            __builtin_amdgcn_sched_barrier(0);
            // Higher issue priority for the matrix and epilogue part of the
            // tile, back to normal for the staging (stores or the wait for
            // the direct loads) and the barrier:
            // when both waves of a SIMD are ready, the one feeding the
            // matrix unit goes first (1-4 % faster on the B=32, K=1024
            // workloads, 1-2 % of it from the ILP-first scheduler the build
            // selects for this unit).
            __builtin_amdgcn_s_setprio(1);
            if constexpr (MAT) mat_store(t, prv);
            const int32_t kb_prv = tile_base(t);
#pragma unroll
            for (int sl = 0; sl < kSlots; ++sl) {
                const int s = sl / RB, rb = sl % RB;
                // The previous tile's epilogue (epi_op, 12 NP steps) is
                // spread evenly over the tile's MFMAs so it issues while the
                // matrix unit works.
                static_for<0, NP>([&](auto Q) {
                    constexpr int q = decltype(Q)::value;
                    cur[rb][q] = M::step(a[sl], xf[q][s], s == 0 ? bv[rb] : cur[rb][q]);
                    if constexpr (!MAT) {
                        constexpr int kMfmas = kSlots * NP;
                        constexpr int kMost = (kEpiSteps + kMfmas - 1) / kMfmas;
                        const int mi = sl * NP + q;
                        const int lo = mi * kEpiSteps / kMfmas, hi = (mi + 1) * kEpiSteps / kMfmas;
                        static_for<0, kMost>([&](auto O) {
                            const int op = lo + decltype(O)::value;
                            if (op < hi) epi_op(prv, op, kb_prv);
                        });
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
                // a[sl] is free: read the fragment needed P slots later
                const int v = sl + P;
                if (v < kSlots)
                    a[v] = frag(b1, v);
                else
                    nx[v - kSlots] = frag(b2, v - kSlots);
                if (sl == kBiasSlot) bias_vec(b2, nbv);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int q = 0; q < P; ++q) a[q] = nx[q];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) bv[rb] = nbv[rb];
            __builtin_amdgcn_s_setprio(0);
            if constexpr (DMA)
                wait_vm<PER + 1>();  // tile t + 3 (issued an iteration ago) has landed
            else
                sstore(b3, st[(i & 1) ^ 1]);
            __syncthreads();
        };
        auto final_epilogue = [&](int t, const floatx4(&sc)[RB][NP]) {
            if constexpr (MAT) {
                mat_store(t, sc);
                return;
            }
            const int32_t kb = tile_base(t);
            static_for<0, kEpiSteps>([&](auto O) { epi_op(sc, decltype(O)::value, kb); });
        };
        int t = 0;
        for (; t + 4 < ntiles; t += 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) iteration(t + i, i);
        }
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

        // ---- merge the four row groups that hold the same point
        // (lexicographic on (score, index)); write labels
#pragma unroll
        for (int np = 0; np < (MAT ? 0 : NP); ++np) {
            float sc = best[np];
            int32_t ix = bidx[np] + 4 * g;
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float so = __shfl_xor(sc, o);
                const int32_t io = __shfl_xor(ix, o);
                if (so > sc || (so == sc && io < ix)) {
                    sc = so;
                    ix = io;
                }
            }
            // |x|^2 for min_dist, from the fragments still in registers
            float xx = 0.f;
            if (min_dist) {
#pragma unroll
                for (int s = 0; s < S; ++s) xx += MS::sumsq(xf[np][s]);
                xx += __shfl_xor(xx, 16);
                xx += __shfl_xor(xx, 32);
            }
            const int64_t j = pbase + np * 16 + col;
            if (g == 0 && j < N) {
                labels[b * N + j] = ix;
                if (min_dist) min_dist[b * N + j] = xx - 2.f * sc;
            }
        }
        // the next item's prologue rewrites the ring, and the workgroup's
        // LDS is released when it ends: no direct load of this item may
        // still be in flight, and no wave may still be reading
        if constexpr (DMA) wait_vm<0>();
        __syncthreads();
    }
}

template <typename T, int S, int NP, bool VEC, bool EXACT, bool SMALLK, int W = kAssignWaves,
          int U = 2>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_assign16(const T* __restrict__ X, const T* __restrict__ C, const float* __restrict__ bias,
                int32_t* __restrict__ labels, float* __restrict__ min_dist, int64_t B, int64_t N,
                int64_t K, int d) {
    assign16_body<T, S, NP, VEC, EXACT, SMALLK, false, W, U>(X, C, bias, labels, min_dist, B, N,
                                                             K, d, nullptr);
}

// The same contraction writing every score (MAT) instead of the argmax.
template <typename T, int S, int NP, bool VEC, bool EXACT, bool SMALLK>
__global__ __launch_bounds__(kAssignWaves * kWave) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_scores16(const T* __restrict__ X, const T* __restrict__ C, const float* __restrict__ bias,
                float* __restrict__ D, int64_t B, int64_t N, int64_t K, int d) {
    assign16_body<T, S, NP, VEC, EXACT, SMALLK, true, kAssignWaves>(X, C, bias, nullptr, nullptr,
                                                                    B, N, K, d, D);
}

// Launch of one instantiation.  W = waves per workgroup; grid_wgs > 0 caps
// the grid at that many workgroups (each then loops over several items).
template <typename T, int S, int NP, bool VEC, bool EXACT, bool SMALLK, bool MAT = false,
          int W = kAssignWaves, int U = 2>
hipError_t launch_assign16_t(const void* X, const void* C, const float* bias, int32_t* labels,
                             float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                             hipStream_t s, float* D = nullptr, int64_t grid_wgs = 0) {
    static_assert(!MAT || W == kAssignWaves, "scores mode uses the default shape");
    constexpr int RC = 4 * S, CHUNKS = kAssignBK * RC;
    constexpr bool DMA = VEC && !SMALLK && CHUNKS % (W * kWave) == 0;
    constexpr int lds = kAssignRing * (kAssignBK * RC * 16 + (DMA ? W * kWave * 4 : kAssignBK * 4));
    static_assert(lds <= kLdsBytes, "LDS budget");
    constexpr int PTS = W * NP * 16;
    const void* kern;
    if constexpr (MAT)
        kern = reinterpret_cast<const void*>(k_scores16<T, S, NP, VEC, EXACT, SMALLK>);
    else
        kern = reinterpret_cast<const void*>(k_assign16<T, S, NP, VEC, EXACT, SMALLK, W, U>);
    static LdsAttr attr;
    hipError_t e = ensure_lds(attr, kern, lds);
    if (e != hipSuccess) return e;
    const int64_t items = B * ((N + PTS - 1) / PTS);
    const dim3 grid((unsigned)(grid_wgs > 0 && grid_wgs < items ? grid_wgs : items));
    if constexpr (MAT)
        hipLaunchKernelGGL((k_scores16<T, S, NP, VEC, EXACT, SMALLK>), grid,
                           dim3(kAssignWaves * kWave), lds, s, static_cast<const T*>(X),
                           static_cast<const T*>(C), bias, D, B, N, K, d);
    else
        hipLaunchKernelGGL((k_assign16<T, S, NP, VEC, EXACT, SMALLK, W, U>), grid, dim3(W * kWave),
                           lds, s, static_cast<const T*>(X), static_cast<const T*>(C), bias,
                           labels, min_dist, B, N, K, d);
    return hipGetLastError();
}

// Estimated VGPRs per lane of k_assign16 with S k-steps and NP point
// blocks: the points' fragments (4 S NP), two accumulator sets of two row
// blocks (16 NP), one tile's centroid fragments (8 S), running and per-tile
// (score, index) pairs (8 NP), and staging, prefetch, bias and addresses
// (about 40).
constexpr int assign16_vgprs(int S, int NP) {
    return 4 * S * NP + 16 * NP + 8 * S + 8 * NP + 40;
}

// Point blocks per wave: the most, up to four, whose register estimate
// stays within 1.3 times the 256 VGPRs a lane has at two waves per SIMD.
// Each centroid fragment read from LDS feeds NP matrix instructions, so
// more is better until spilling dominates: a moderate overflow spills
// loop-invariant point fragments to scratch (cached), which costs less than
// halving the matrix work per fragment, while eight blocks overflow by far.
// Measured on B=32, N=65536, K=1024 fp16 (every shape, same process): at
// d = 256 four blocks spill 129 registers and run 10 % faster than two,
// which fit; eight blocks spill 550-700 registers at d = 64-256 and run
// level with four at d = 64, 4x and 6x slower at d = 128 and 256.  Gives
// 4 for every S <= 8.
constexpr int assign16_np(int S) {
    return assign16_vgprs(S, 4) * 10 <= 256 * 13   ? 4
           : assign16_vgprs(S, 2) * 10 <= 256 * 13 ? 2
                                                   : 1;
}

// Waves per workgroup: four, so two workgroups share a CU, each with its
// own LDS ring, and one workgroup's barrier waits overlap the other's
// matrix work (eight waves, one workgroup per CU, measured 8-28 % slower
// with four point blocks at d = 64, 128 and 256; two waves, four
// workgroups per CU, each staging every centroid tile for half the points,
// 2-11 % slower at d = 64 and 128 and 67 % at d = 256).
constexpr int assign16_waves(int) { return 4; }

// Whether 16-bit rows of d dimensions take the register-resident kernel:
// up to 256 dimensions in whole 16-byte chunks, or up to 128 otherwise.
// Rows of 129-256 dimensions that are not whole chunks need eight k-steps
// of point fragments plus the unit offsets of the staged tiles, which spill
// about 900 bytes per lane; the split-d kernel, which keeps no point rows
// in registers, runs them 2.4-3.2 times faster (B=8, N=65536, K=1024, same
// labels: d = 228 fp16 1.230 -> 0.402 ms, d = 129 fp16 1.907 -> 0.649 ms).
constexpr bool assign16_resident(int d) { return d <= 128 || (d <= 256 && d % 8 == 0); }

// 16-bit inputs with d <= 256: S = k-steps of 32 (a power of two covering
// d), assign16_np(S) 16-point blocks per wave, assign16_waves(S) waves.
template <typename T>
hipError_t dispatch_assign16(const void* X, const void* C, const float* bias, int32_t* labels,
                             float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                             hipStream_t s) {
    const int need = (d + 31) / 32;
    const bool vec = (d % 8) == 0;
#define FK_ASSIGN16_CASE(SS)                                                                   \
    if (need <= SS) {                                                                          \
        constexpr int NPP = assign16_np(SS), WW = assign16_waves(SS);                          \
        if (K < kAssignBK)                                                                     \
            return vec ? launch_assign16_t<T, SS, NPP, true, false, true, false, WW>(          \
                             X, C, bias, labels, min_dist, B, N, K, d, s)                      \
                       : launch_assign16_t<T, SS, NPP, false, false, true, false, WW>(         \
                             X, C, bias, labels, min_dist, B, N, K, d, s);                     \
        if (vec && d == 32 * SS)                                                               \
            return launch_assign16_t<T, SS, NPP, true, true, false, false, WW>(                \
                X, C, bias, labels, min_dist, B, N, K, d, s);                                  \
        if (vec)                                                                               \
            return launch_assign16_t<T, SS, NPP, true, false, false, false, WW>(               \
                X, C, bias, labels, min_dist, B, N, K, d, s);                                  \
        if (d % 4 == 0)                                                                        \
            return launch_assign16_t<T, SS, NPP, false, false, false, false, WW, 8>(           \
                X, C, bias, labels, min_dist, B, N, K, d, s);                                  \
        if (d % 2 == 0)                                                                        \
            return launch_assign16_t<T, SS, NPP, false, false, false, false, WW, 4>(           \
                X, C, bias, labels, min_dist, B, N, K, d, s);                                  \
        return launch_assign16_t<T, SS, NPP, false, false, false, false, WW, 2>(               \
            X, C, bias, labels, min_dist, B, N, K, d, s);                                      \
    }
    FK_ASSIGN16_CASE(1)
    FK_ASSIGN16_CASE(2)
    FK_ASSIGN16_CASE(4)
    FK_ASSIGN16_CASE(8)
#undef FK_ASSIGN16_CASE
    return hipErrorInvalidValue;
}

// All scores x.c + bias into D [B][N][K] fp32, d <= 256 (same contraction,
// tiles and dispatch as dispatch_assign16).
template <typename T>
hipError_t dispatch_scores16(const void* X, const void* C, const float* bias, float* D, int64_t B,
                             int64_t N, int64_t K, int d, hipStream_t s) {
    const int need = (d + 31) / 32;
    const bool vec = (d % 8) == 0;
#define FK_SCORES16_CASE(SS, NPP)                                                                \
    if (need <= SS) {                                                                            \
        if (K < kAssignBK)                                                                       \
            return vec ? launch_assign16_t<T, SS, NPP, true, false, true, true>(                 \
                             X, C, bias, nullptr, nullptr, B, N, K, d, s, D)                     \
                       : launch_assign16_t<T, SS, NPP, false, false, true, true>(                \
                             X, C, bias, nullptr, nullptr, B, N, K, d, s, D);                    \
        return vec ? launch_assign16_t<T, SS, NPP, true, false, false, true>(                    \
                         X, C, bias, nullptr, nullptr, B, N, K, d, s, D)                         \
                   : launch_assign16_t<T, SS, NPP, false, false, false, true>(                   \
                         X, C, bias, nullptr, nullptr, B, N, K, d, s, D);                        \
    }
    FK_SCORES16_CASE(1, assign16_np(1))
    FK_SCORES16_CASE(2, assign16_np(2))
    FK_SCORES16_CASE(4, assign16_np(4))
    FK_SCORES16_CASE(8, assign16_np(8))
#undef FK_SCORES16_CASE
    return hipErrorInvalidValue;
}

static_assert(assign16_np(1) == 4 && assign16_np(2) == 4 && assign16_np(4) == 4 &&
                  assign16_np(8) == 4,
              "point blocks per wave");
static_assert(assign16_waves(4) == 4 && assign16_waves(8) == 4, "waves per workgroup");

}  // namespace
}  // namespace fk
