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
//  * The argsort is a counting sort, since keys are small integers in [0, K).
//    Tiled form (K <= 16000 and a per-tile table of modest size): each
//    workgroup histograms a tile of 4096 labels in LDS and writes the tile's
//    counts; a column pass turns them into per-tile prefix counts; the
//    scatter workgroup gives every label of its tile a base position from
//    them and ranks its elements by lane order within each wave (ballots),
//    so no global atomics are needed.  Larger K: counts from a histogram
//    with global atomics and the argsort from least-significant-digit radix
//    passes over 8-bit digits.  Both forms are stable: inside a segment the
//    points keep increasing index order.
//  * The gather-reduce gives every wave a fixed run of 256 sorted positions,
//    so hot clusters spread over many waves.  The segment walk is
//    wave-uniform (row indices come through readlane, segment boundaries
//    from a window of offsets held in one VGPR), lanes split the d
//    dimensions of each row, and rows are loaded a batch at a time for
//    memory-level parallelism.
//  * Fused finalize: a segment that lies inside one wave's run is finalized
//    from registers; otherwise each piece adds its partial sum with one row
//    of fp32 atomics and bumps the segment's arrival counter, and the last
//    piece to arrive reads the total back and finalizes it.  Finalize divides
//    by the exact integer count (IEEE fp32 division), writes the
//    round-to-nearest-even copy in the input dtype with its |c|^2 bias for
//    the next assignment, and tracks the largest squared centroid move;
//    empty segments keep the previous centroid bit for bit.
#include <math.h>

#include "fk_internal.h"

namespace fk {
namespace {

constexpr int kBlock = 256;
constexpr int kSortTile = 4096;          // labels per histogram / scatter workgroup
constexpr int kSortPer = kSortTile / kBlock;  // labels per thread of a sort tile
constexpr int64_t kLdsBinsMax = 16384;   // LDS-privatised bins (64 KiB)
constexpr int64_t kTiledBinsMax = 16000; // tiled sort: bins + scan scratch stay under 64 KiB

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T>
__device__ inline float to_f32(T v) {
    return (float)v;
}

// Canonical order of a centroid row's squared norm: lane l adds the E
// consecutive elements l E .. l E + E - 1 (E = the smallest power of two
// with 64 E >= d) in order, then the wave adds the 64 partial sums by the
// butterfly of wave_sum.  Every kernel that writes a centroid bias follows
// it (the segment sums hold exactly these elements per lane), so the bias
// has the same bits whichever kernel wrote it.
__device__ inline int row_part(int d) {
    int e = 1;
    while (e * kWave < d) e <<= 1;
    return e;
}

// ---------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void k_add_f32(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] += src[i];
}

__global__ void k_add_i32(int32_t* __restrict__ dst, const int32_t* __restrict__ src, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] += src[i];
}

// Zeroes up to four 32-bit ranges in one launch (the grid strides over each).
struct ZeroRanges {
    uint32_t* p[4];
    int64_t n[4];
};
__global__ void k_zero(ZeroRanges z) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        for (int64_t i = i0; i < z.n[r]; i += stride) z.p[r][i] = 0u;
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
    const int E = row_part(d);
    float s = 0.f;
    for (int e = 0; e < E; ++e) {
        const int j = lane * E + e;
        if (j >= d) break;
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
    const int E = row_part(d);
    for (int e = 0; e < E; ++e) {
        const int j = lane * E + e;
        if (j >= d) break;
        const T q = (T)C[row * d + j];
        lowp[row * d + j] = q;
        const float v = to_f32(q);
        s = fmaf(v, v, s);
    }
    s = wave_sum(s);
    if (lane == 0) bias[row] = -0.5f * s;
}

// ---------------------------------------------------------------------------
// Pieces of the segment sums: every nonempty segment [off[k], off[k+1]) is
// cut into pieces of at most kSegRun sorted positions, one wave each.  The
// piece block of a problem holds P[0] = number of pieces, P[1 + j] = the
// segment of piece j (-1 in the unused slots up to the capacity M) and
// P[1 + M + j] = its first position; poff[k] is the first piece of
// segment k.
__device__ inline int32_t npieces_of(int32_t count) { return (count + kSegRun - 1) / kSegRun; }

// Clears the sum rows and arrival counters of the segments with more than
// one piece (the only rows the segment sums accumulate into): workgroup wg
// of nwg takes every nwg-th group of rows, one wave per row.  Each wave
// tests 64 of its rows at once (one load per lane) and clears those that
// need it, so the tests cost one round trip, not one per row.
__device__ inline void clear_multi_rows(const int32_t* __restrict__ counts,
                                        float* __restrict__ sums, int32_t* __restrict__ arrive,
                                        int64_t K, int64_t d, int64_t wg, int64_t nwg) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = blockDim.x / kWave;
    const int64_t stride = nwg * nw;
    const int64_t k0 = wg * nw + threadIdx.x / kWave;  // this wave's rows: k0 + r stride
    for (int64_t r0 = 0; k0 + r0 * stride < K; r0 += kWave) {
        const int64_t k = k0 + (r0 + lane) * stride;
        uint64_t m = __ballot(k < K && counts[k] > kSegRun);
        while (m) {
            const int64_t kk = k0 + (r0 + __ffsll((unsigned long long)m) - 1) * stride;
            m &= m - 1;
            float* row = sums + kk * d;
            for (int64_t c = lane; c < d; c += kWave) row[c] = 0.f;
            if (lane == 0) arrive[kk] = 0;
        }
    }
}

// The plan workgroup: 16 waves, 4 labels per thread (fewer serial label
// steps per thread than 4 waves with 16 each; one workgroup is all a
// problem with K <= 4096 gets)
constexpr int kPlanThreads = 1024;
constexpr int kPlanPer = 4;
constexpr int kPlanBlock = kPlanThreads * kPlanPer;  // labels per plan workgroup
static_assert(kPlanBlock == kPlanLabels, "plan block size");

// ---- tiled counting sort ----------------------------------------------------
// th[b][t][k] = #{i in tile t : labels[b][i] == k}, th[b][t][K] = labels out
// of [0, K) in the tile.
__global__ __launch_bounds__(kBlock) void k_tile_hist(const int32_t* __restrict__ labels,
                                                      int32_t* __restrict__ th, int64_t N,
                                                      int64_t K, int64_t T) {
    extern __shared__ int32_t s_hist[];  // [K + 1]
    const int64_t b = blockIdx.y;
    const int64_t t = blockIdx.x;
    const int64_t i0 = t * kSortTile;
    const int64_t i1 = min(i0 + (int64_t)kSortTile, N);
    const int32_t* lab = labels + b * N;
    // all label loads first, so they are in flight together (and while the
    // bins are cleared)
    int32_t a[kSortPer];
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        const int64_t i = i0 + threadIdx.x + j * kBlock;
        a[j] = i < i1 ? lab[i] : 0;
    }
    for (int64_t k = threadIdx.x; k <= K; k += kBlock) s_hist[k] = 0;
    __syncthreads();
    int32_t bad = 0;
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        if (i0 + threadIdx.x + j * kBlock < i1) {
            if (a[j] >= 0 && a[j] < K)
                atomicAdd(&s_hist[a[j]], 1);
            else
                ++bad;
        }
    }
    if (bad) atomicAdd(&s_hist[K], bad);
    __syncthreads();
    int32_t* out = th + (b * T + t) * (K + 1);
    for (int64_t k = threadIdx.x; k <= K; k += kBlock) out[k] = s_hist[k];
}

// Column pass: th[b][t][k] <- sum_{t' < t} th[b][t'][k]; counts[b][k] and
// bad[b] (column K) receive the column totals.  A workgroup takes 64
// columns; its G waves split the tiles into G consecutive groups, sum their
// group, exchange the group totals through LDS and rewrite their group as a
// running prefix.  Each wave walks its tiles in dependent batches, so many
// tiles per problem (one problem of 2^20 points: 256 tiles) want more
// waves per column block.
template <int G>
__global__ __launch_bounds__(G * kWave) void k_tile_colscan(int32_t* __restrict__ th,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ bad, int64_t K,
                                                            int64_t T) {
    constexpr int kColGroups = G;
    __shared__ int32_t s_tot[kColGroups][kWave];
    const int64_t b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = threadIdx.x / kWave;
    const int64_t k = (int64_t)blockIdx.x * kWave + lane;
    const int64_t per = (T + kColGroups - 1) / kColGroups;
    const int64_t t0 = min(g * per, T), t1 = min(t0 + per, T);
    int32_t* col = th + b * T * (K + 1) + min(k, K);
    // both passes load kColBatch tiles at once: whole batches, then the
    // tail as one masked batch
    constexpr int kColBatch = 8;
    int32_t sum = 0;
    if (k <= K) {
        int64_t t = t0;
        for (; t + kColBatch <= t1; t += kColBatch) {
            int32_t v[kColBatch];
#pragma unroll
            for (int u = 0; u < kColBatch; ++u) v[u] = col[(t + u) * (K + 1)];
#pragma unroll
            for (int u = 0; u < kColBatch; ++u) sum += v[u];
        }
        if (t < t1) {
            int32_t v[kColBatch];
#pragma unroll
            for (int u = 0; u < kColBatch; ++u) v[u] = t + u < t1 ? col[(t + u) * (K + 1)] : 0;
#pragma unroll
            for (int u = 0; u < kColBatch; ++u) sum += v[u];
        }
    }
    s_tot[g][lane] = sum;
    __syncthreads();
    int32_t run = 0, total = 0;
#pragma unroll
    for (int q = 0; q < kColGroups; ++q) {
        run += q < g ? s_tot[q][lane] : 0;
        total += s_tot[q][lane];
    }
    if (k > K) return;
    int64_t t = t0;
    for (; t + kColBatch <= t1; t += kColBatch) {
        int32_t v[kColBatch];
#pragma unroll
        for (int u = 0; u < kColBatch; ++u) v[u] = col[(t + u) * (K + 1)];
#pragma unroll
        for (int u = 0; u < kColBatch; ++u) {
            col[(t + u) * (K + 1)] = run;
            run += v[u];
        }
    }
    if (t < t1) {
        int32_t v[kColBatch];
#pragma unroll
        for (int u = 0; u < kColBatch; ++u) v[u] = t + u < t1 ? col[(t + u) * (K + 1)] : 0;
#pragma unroll
        for (int u = 0; u < kColBatch; ++u) {
            if (t + u < t1) col[(t + u) * (K + 1)] = run;
            run += v[u];
        }
    }
    if (g == 0) {
        if (k < K)
            counts[b * K + k] = total;
        else
            bad[b] = total;
    }
}

// Plan, part 1 (only when K > kPlanBlock): totals of counts and pieces of
// every block of kPlanBlock labels.
__global__ __launch_bounds__(kBlock) void k_plan_totals(const int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ part, int64_t K) {
    __shared__ int32_t s_red[2][kBlock];
    const int64_t b = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const int64_t k0 = blk * kPlanBlock;
    int32_t c = 0, p = 0;
    for (int64_t k = k0 + threadIdx.x; k < min(k0 + kPlanBlock, K); k += kBlock) {
        const int32_t v = counts[b * K + k];
        c += v;
        p += npieces_of(v);
    }
    s_red[0][threadIdx.x] = c;
    s_red[1][threadIdx.x] = p;
    __syncthreads();
    for (int o = kBlock / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            s_red[0][threadIdx.x] += s_red[0][threadIdx.x + o];
            s_red[1][threadIdx.x] += s_red[1][threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        part[(b * nblk + blk) * 2 + 0] = s_red[0][0];
        part[(b * nblk + blk) * 2 + 1] = s_red[1][0];
    }
}

// Inclusive scan of v over the NT threads of the workgroup in thread order
// (wave scans by lane shifts, then the wave totals through LDS); *total
// receives the sum over the workgroup.  Every thread must call it.
template <int NT>
__device__ inline int32_t block_inclusive_scan(int32_t v, int32_t* __restrict__ s_w,
                                               int32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int32_t t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    if (lane == kWave - 1) s_w[w] = v;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int q = 0; q < NT / kWave; ++q) {
        const int32_t t = s_w[q];
        before += q < w ? t : 0;
        all += t;
    }
    __syncthreads();  // s_w may be reused
    *total = all;
    return before + v;
}

// Plan, part 2: for block blk of kPlanBlock labels of problem b, the
// offsets (exclusive scan of the counts) and first pieces, then every piece
// of the block's segments.  Thread t owns the kPlanPer consecutive labels
// kPlanPer t .. kPlanPer t + kPlanPer - 1 of the block in registers for the
// scans (each a scan of the per-thread totals); the results go through LDS
// so that thread t then writes labels t, t + kPlanThreads, ...  A segment of few
// pieces is written by the thread that holds it; the pieces of segments with many
// (hot clusters) are listed, numbered with a second scan, and split evenly
// over the threads (each walks a contiguous run of them).  The last block
// writes the totals; block 0 of problem 0 clears the move word.
__global__ __launch_bounds__(kPlanThreads) void k_plan(const int32_t* __restrict__ counts,
                                                 const int32_t* __restrict__ part,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ poff,
                                                 int32_t* __restrict__ pieces,
                                                 uint32_t* __restrict__ move, int64_t K,
                                                 int64_t M) {
    constexpr int kBigPieces = 8;  // segments with more pieces go to the shared list
    __shared__ int32_t s_w[kPlanThreads / kWave];
    __shared__ int32_t s_base[2];
    __shared__ int32_t s_off[kPlanBlock];
    __shared__ int32_t s_po[kPlanBlock];
    __shared__ int32_t s_big_k[kPlanThreads], s_big_pos[kPlanThreads], s_big_piece[kPlanThreads],
        s_big_first[kPlanThreads + 1];
    __shared__ int32_t s_nbig;
    const int64_t b = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const int64_t k0 = blk * kPlanBlock;
    const int n = (int)min((int64_t)kPlanBlock, K - k0);
    if (threadIdx.x < 2) {
        int32_t acc = 0;
        for (int64_t q = 0; q < blk; ++q) acc += part[(b * nblk + q) * 2 + threadIdx.x];
        s_base[threadIdx.x] = acc;
    }
    if (threadIdx.x == 0) s_nbig = 0;
    const int i0 = threadIdx.x * kPlanPer;
    int32_t c[kPlanPer];
    int32_t cs = 0, ps = 0;
#pragma unroll
    for (int u = 0; u < kPlanPer; ++u) {
        c[u] = i0 + u < n ? counts[b * K + k0 + i0 + u] : 0;
        cs += c[u];
        ps += npieces_of(c[u]);
    }
    // exclusive starts of this thread's labels and pieces within the block
    int32_t tot_c, tot_p;
    const int32_t ic = block_inclusive_scan<kPlanThreads>(cs, s_w, &tot_c);
    const int32_t ip = block_inclusive_scan<kPlanThreads>(ps, s_w, &tot_p);
    const int32_t bc = s_base[0], bp = s_base[1];
    int32_t* off = offsets + b * (K + 1);
    int32_t* po = poff + b * (K + 1);
    int32_t* P = pieces + b * (2 * M + 1);
    // offsets and first pieces through LDS, so the stores below go out in
    // label order across the lanes (coalesced)
    int32_t ro = bc + ic - cs, rp = bp + ip - ps;  // running offset and first piece
#pragma unroll
    for (int u = 0; u < kPlanPer; ++u) {
        if (i0 + u < n) {
            s_off[i0 + u] = ro;
            s_po[i0 + u] = rp;
            ro += c[u];
            rp += npieces_of(c[u]);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kPlanThreads) {
        const int64_t k = k0 + i;
        const int32_t o0 = s_off[i], p0 = s_po[i];
        off[k] = o0;
        po[k] = p0;
        const int32_t pc = (i + 1 < n ? s_po[i + 1] : bp + tot_p) - p0;
        bool mine = pc <= kBigPieces;
        if (!mine) {
            const int32_t at = atomicAdd(&s_nbig, 1);
            if (at < kPlanThreads) {
                s_big_k[at] = (int32_t)k;
                s_big_pos[at] = o0;
                s_big_piece[at] = p0;
                s_big_first[at] = pc;  // piece count until the scan below
            } else {
                mine = true;  // list full: write them here
            }
        }
        if (mine)
            for (int32_t q = 0; q < pc; ++q) {
                P[1 + p0 + q] = (int32_t)k;
                P[1 + M + p0 + q] = o0 + q * kSegRun;
            }
    }
    if (blk == nblk - 1) {
        if (threadIdx.x == 0) {
            off[K] = bc + tot_c;
            po[K] = bp + tot_p;
            P[0] = bp + tot_p;
        }
        // unused slots: a segment-sums wave may read its slot without
        // waiting for the count
        for (int64_t j = bp + tot_p + threadIdx.x; j < M; j += kPlanThreads) P[1 + j] = -1;
    }
    __syncthreads();
    const int nbig = min(s_nbig, kPlanThreads);
    if (nbig > 0) {
        // number the listed pieces: entry r owns flat pieces
        // s_big_first[r] .. s_big_first[r + 1] - 1
        const int32_t mine = (int)threadIdx.x < nbig ? s_big_first[threadIdx.x] : 0;
        int32_t tb;
        const int32_t inc = block_inclusive_scan<kPlanThreads>(mine, s_w, &tb);
        if ((int)threadIdx.x < nbig) s_big_first[threadIdx.x] = inc - mine;
        if (threadIdx.x == 0) s_big_first[nbig] = tb;
        __syncthreads();
        // thread t writes flat pieces [t tb / NT, (t + 1) tb / NT)
        const int32_t j0 = (int32_t)((int64_t)threadIdx.x * tb / kPlanThreads);
        const int32_t j1 = (int32_t)((int64_t)(threadIdx.x + 1) * tb / kPlanThreads);
        if (j0 < j1) {
            int lo = 0, hi = nbig - 1;  // last entry whose first piece is <= j0
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_big_first[mid] <= j0)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            int r = lo;
            int32_t rend = s_big_first[r + 1];
            for (int32_t j = j0; j < j1; ++j) {
                while (j >= rend) rend = s_big_first[++r + 1];
                const int32_t q = j - s_big_first[r];
                P[1 + s_big_piece[r] + q] = s_big_k[r];
                P[1 + M + s_big_piece[r] + q] = s_big_pos[r] + q * kSegRun;
            }
        }
    }
    if (b == 0 && blk == 0 && threadIdx.x == 0 && move) *move = 0u;
}

// Workgroup -> (problem b, tile t) of the scatter.  Workgroups go to the 8
// XCDs round-robin (workgroup g to XCD g mod 8).  With pairs = B T > 0 (1-D
// grid of 8 ceil(B T / 8) workgroups) the (b, t) pairs, problem-major, are
// cut into 8 consecutive runs, one per XCD, so each XCD scatters
// consecutive tiles of a problem: neighbouring tiles write neighbouring
// positions inside every segment, so the cache lines they share are
// completed in one L2 and written back once instead of once per XCD
// (K = 4096 over N = 2^20 in one problem: 36 MB written for 4 MB of
// indices with the plain order).  pairs = 0: 2-D grid (tiles, B).  Returns
// false for the padding workgroups past the last pair.
__device__ inline bool scatter_tile(int64_t pairs, int64_t T, int64_t& b, int64_t& t) {
    if (pairs == 0) {
        b = blockIdx.y;
        t = blockIdx.x;
        return true;
    }
    const int64_t run = (pairs + 7) / 8;
    const int64_t L = (int64_t)(blockIdx.x % 8) * run + blockIdx.x / 8;
    b = L / T;
    t = L % T;
    return L < pairs;
}

// Scatter of tile t: base of label k = offsets[k] + th[b][t][k].  The
// scatter is stable: a label's points land in increasing index order.
// Round j takes elements i0 + 256 j + tid (64 consecutive per wave); inside
// a wave, the lanes holding the same label are found with one ballot per
// label bit (nbits bits cover K - 1) and ranked by lane; across the waves
// of a round each label's LDS base is advanced wave by wave, with a barrier
// between, by the lowest lane of each group.  With sums the workgroups also
// clear the sum rows of multi-piece segments.
__global__ __launch_bounds__(kBlock) void k_tile_scatter(
    const int32_t* __restrict__ labels, const int32_t* __restrict__ th,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_idx,
    const int32_t* __restrict__ counts, float* __restrict__ sums, int32_t* __restrict__ arrive,
    int64_t N, int64_t K, int64_t T, int64_t d, int64_t pairs, int nbits) {
    extern __shared__ int32_t s_base[];  // [K]
    int64_t b, t;
    if (!scatter_tile(pairs, T, b, t)) return;
    if (sums) clear_multi_rows(counts + b * K, sums + b * K * d, arrive + b * K, K, d, t, T);
    const int32_t* pre = th + (b * T + t) * (K + 1);
    const int32_t* off = offsets + b * (K + 1);
    for (int64_t k = threadIdx.x; k < K; k += kBlock) s_base[k] = off[k] + pre[k];
    __syncthreads();
    const int64_t i0 = t * kSortTile;
    const int64_t i1 = min(i0 + (int64_t)kSortTile, N);
    const int32_t* lab = labels + b * N;
    int32_t* out = sorted_idx + b * N;
    int32_t a[kSortPer];
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        const int64_t i = i0 + threadIdx.x + j * kBlock;
        a[j] = i < i1 ? lab[i] : -1;
    }
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint64_t below = lane ? ~0ull >> (64 - lane) : 0ull;
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        const int64_t i = i0 + threadIdx.x + j * kBlock;
        const int32_t v = a[j];
        const bool valid = v >= 0 && v < K;
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (v >> bit) & 1;
            const uint64_t m = __ballot(on);
            peers &= on ? m : ~m;
        }
        if (!valid) peers = 0;
        const int rank = __popcll(peers & below);
        int32_t base = 0;
        for (int w = 0; w < kBlock / kWave; ++w) {
            if (wave == w && valid && rank == 0) base = atomicAdd(&s_base[v], __popcll(peers));
            __syncthreads();
        }
        base = __shfl(base, valid ? __ffsll((unsigned long long)peers) - 1 : lane);
        if (valid) out[base + rank] = (int32_t)i;
    }
}

// The same scatter for K <= kWaveBinsMax without barriers between the
// waves: each of the NW waves of the workgroup takes kSortTile / NW
// consecutive elements of the tile, in rounds of 64.  A first pass counts
// each wave's labels (the 16-bit counts of waves 2j and 2j+1 share the
// 32-bit LDS word j of the label), the counts become per-wave exclusive
// prefixes, and a second pass ranks each round's lanes by ballot match and
// advances the wave's own 16-bit cursor with one LDS atomic per label group;
// the waves' ranges and the rounds inside a wave are in index order, so the
// scatter is stable.  More waves mean fewer dependent rounds per wave (a
// round is a chain of ballots, an LDS atomic and a shuffle).
constexpr int64_t kWaveBinsMax = 4096;
constexpr int kScatterWaves = 16;
template <int NW>
constexpr int scatter_w_lds(int64_t K) {
    return (int)((1 + NW / 2) * K * (int64_t)sizeof(int32_t));
}
template <int NW>
__global__ __launch_bounds__(NW * kWave) void k_tile_scatter_w(
    const int32_t* __restrict__ labels, const int32_t* __restrict__ th,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_idx,
    const int32_t* __restrict__ counts, float* __restrict__ sums, int32_t* __restrict__ arrive,
    int64_t N, int64_t K, int64_t T, int64_t d, int64_t pairs, int nbits) {
    constexpr int kRange = kSortTile / NW;  // elements per wave
    constexpr int kPer = kRange / kWave;    // rounds per wave
    static_assert(NW % 2 == 0 && kRange % kWave == 0 && kRange < 65536, "16-bit cursors");
    extern __shared__ int32_t s_mem[];  // base [K] | cursor word j of every label [NW/2][K]
    int32_t* s_base = s_mem;
    uint32_t* s_cur = reinterpret_cast<uint32_t*>(s_mem + K);
    int64_t b, t;
    if (!scatter_tile(pairs, T, b, t)) return;
    const int32_t* pre = th + (b * T + t) * (K + 1);
    const int32_t* off = offsets + b * (K + 1);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t w0 = t * kSortTile + (int64_t)wave * kRange;
    const int64_t i1 = min(t * kSortTile + (int64_t)kSortTile, N);
    const int32_t* lab = labels + b * N;
    int32_t* out = sorted_idx + b * N;
    uint32_t* cur = s_cur + (wave >> 1) * K;
    const uint32_t sh = 16u * (uint32_t)(wave & 1);
    // every global load first, so they share one round trip: this wave's
    // labels, the bases of the labels this thread initialises, and the
    // counts the row clearing tests
    int32_t a[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = w0 + j * kWave + lane;
        a[j] = i < i1 ? lab[i] : -1;
    }
    constexpr int kBasesPer = (int)((kWaveBinsMax + NW * kWave - 1) / (NW * kWave));
    int32_t base[kBasesPer];
#pragma unroll
    for (int q = 0; q < kBasesPer; ++q) {
        const int64_t k = threadIdx.x + (int64_t)q * NW * kWave;
        const int64_t kc = min(k, K - 1);  // unconditional loads: no wait per label
        const int32_t v = off[kc] + pre[kc];
        base[q] = k < K ? v : 0;
    }
    if (sums) clear_multi_rows(counts + b * K, sums + b * K * d, arrive + b * K, K, d, t, T);
#pragma unroll
    for (int q = 0; q < kBasesPer; ++q) {
        const int64_t k = threadIdx.x + (int64_t)q * NW * kWave;
        if (k < K) {
            s_base[k] = base[q];
#pragma unroll
            for (int j = 0; j < NW / 2; ++j) s_cur[j * K + k] = 0u;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (a[j] >= 0 && a[j] < K) atomicAdd(&cur[a[j]], 1u << sh);
    __syncthreads();
    // counts -> exclusive prefixes over the waves, in wave order
    // (all words of a label read before any is rewritten: one LDS round
    // trip instead of one per word)
    for (int64_t k = threadIdx.x; k < K; k += NW * kWave) {
        uint32_t c[NW / 2];
#pragma unroll
        for (int j = 0; j < NW / 2; ++j) c[j] = s_cur[j * K + k];
        uint32_t run = 0;
#pragma unroll
        for (int j = 0; j < NW / 2; ++j) {
            const uint32_t lo = c[j] & 0xffffu;
            s_cur[j * K + k] = run | ((run + lo) << 16);
            run += lo + (c[j] >> 16);
        }
    }
    __syncthreads();
    const uint64_t below = lane ? ~0ull >> (64 - lane) : 0ull;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = w0 + j * kWave + lane;
        const int32_t v = a[j];
        const bool valid = v >= 0 && v < K;
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (v >> bit) & 1;
            const uint64_t m = __ballot(on);
            peers &= on ? m : ~m;
        }
        if (!valid) peers = 0;
        const int rank = __popcll(peers & below);
        uint32_t old = 0;
        if (valid && rank == 0) old = atomicAdd(&cur[v], (uint32_t)__popcll(peers) << sh);
        old = __shfl(old, valid ? __ffsll((unsigned long long)peers) - 1 : lane);
        if (valid) out[s_base[v] + (int32_t)((old >> sh) & 0xffffu) + rank] = (int32_t)i;
    }
}

// ---- counting sort with global atomics (large K) ----------------------------
// counts[b][k] += #{i in tile : labels[b][i] == k}; labels out of [0, K) are
// counted in bad[b] and skipped.
__global__ __launch_bounds__(kBlock) void k_histogram(const int32_t* __restrict__ labels,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ bad, int64_t N,
                                                      int64_t K, int use_lds) {
    extern __shared__ int32_t s_hist[];
    const int64_t b = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * kSortTile;
    const int64_t i1 = min(i0 + (int64_t)kSortTile, N);
    const int32_t* lab = labels + b * N;
    int32_t* cnt = counts + b * K;
    int32_t nbad = 0;
    if (use_lds) {
        for (int64_t k = threadIdx.x; k < K; k += kBlock) s_hist[k] = 0;
        __syncthreads();
        for (int64_t i = i0 + threadIdx.x; i < i1; i += kBlock) {
            const int32_t a = lab[i];
            if (a >= 0 && a < K)
                atomicAdd(&s_hist[a], 1);
            else
                ++nbad;
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
                ++nbad;
        }
    }
    if (nbad) atomicAdd(&bad[b], nbad);
}

// ---- radix argsort (K above the tiled sort's limit) ---------------------------
// A least-significant-digit radix sort of the valid labels by 8-bit digits,
// each pass a stable counting sort of (label, point) pairs, so the result
// is the stable argsort for any K.  Pass 0 reads the labels (skipping those
// outside [0, K)) with the point index as value; later passes read the
// previous pass's pairs, of which there are nvalid[b].
constexpr int kDigits = 256;

// dth[b][t][r] = #{elements of tile t whose digit is r}
__global__ __launch_bounds__(kBlock) void k_digit_hist(const int32_t* __restrict__ keys,
                                                       int64_t key_stride, int64_t N, int64_t K,
                                                       int first,
                                                       const int32_t* __restrict__ nvalid,
                                                       int shift, int32_t* __restrict__ dth,
                                                       int64_t T) {
    __shared__ int32_t s_h[kDigits];
    const int64_t b = blockIdx.y, t = blockIdx.x;
    s_h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t n = first ? N : nvalid[b];
    const int64_t i0 = t * kSortTile;
    const int64_t i1 = min(i0 + (int64_t)kSortTile, n);
    const int32_t* kin = keys + b * key_stride;
    int32_t a[kSortPer];
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        const int64_t i = i0 + threadIdx.x + j * kBlock;
        a[j] = i < i1 ? kin[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        const int64_t i = i0 + threadIdx.x + j * kBlock;
        if (i < i1 && a[j] >= 0 && a[j] < K) atomicAdd(&s_h[(a[j] >> shift) & (kDigits - 1)], 1);
    }
    __syncthreads();
    dth[(b * T + t) * kDigits + threadIdx.x] = s_h[threadIdx.x];
}

// dth[b][t][r] <- (elements of digit < r) + (elements of digit r in tiles
// < t): the output base of each tile and digit; nvalid[b] = total.  One
// workgroup of 4 x 256 threads per problem: thread (g, r) takes digit r over
// the g-th quarter of the tiles.
constexpr int kDigitGroups = 4;
__global__ __launch_bounds__(kDigits * kDigitGroups) void k_digit_colscan(
    int32_t* __restrict__ dth, int32_t* __restrict__ nvalid, int64_t T) {
    __shared__ int32_t s_tot[kDigitGroups][kDigits];
    __shared__ int32_t s_scan[kDigits];
    const int64_t b = blockIdx.x;
    const int r = threadIdx.x & (kDigits - 1);
    const int g = threadIdx.x / kDigits;
    const int64_t per = (T + kDigitGroups - 1) / kDigitGroups;
    const int64_t t0 = min(g * per, T), t1 = min(t0 + per, T);
    int32_t* col = dth + b * T * kDigits + r;
    int32_t sum = 0;
    int64_t t = t0;
    for (; t + 8 <= t1; t += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = col[(t + u) * kDigits];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; t < t1; ++t) sum += col[t * kDigits];
    s_tot[g][r] = sum;
    __syncthreads();
    int32_t run = 0, total = 0;
#pragma unroll
    for (int q = 0; q < kDigitGroups; ++q) {
        run += q < g ? s_tot[q][r] : 0;
        total += s_tot[q][r];
    }
    // inclusive scan of the digit totals (Hillis-Steele over 256 entries)
    if (g == 0) s_scan[r] = total;
    __syncthreads();
    for (int off = 1; off < kDigits; off <<= 1) {
        const int32_t v = (g == 0 && r >= off) ? s_scan[r - off] : 0;
        __syncthreads();
        if (g == 0) s_scan[r] += v;
        __syncthreads();
    }
    run += s_scan[r] - total;
    if (threadIdx.x == 0) nvalid[b] = s_scan[kDigits - 1];
    t = t0;
    for (; t + 8 <= t1; t += 8) {
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = col[(t + u) * kDigits];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            col[(t + u) * kDigits] = run;
            run += v[u];
        }
    }
    for (; t < t1; ++t) {
        const int32_t v = col[t * kDigits];
        col[t * kDigits] = run;
        run += v;
    }
}

// Stable scatter of one pass: element i of tile t goes to
// dth[b][t][digit] + (its rank among the tile's elements of that digit, in
// index order), with wave-private cursors as in k_tile_scatter_w (wave w of
// four takes 1024 consecutive elements; two waves' 16-bit counts share a
// word).
constexpr int kWaveRange = kSortTile / (kBlock / kWave);  // elements per wave
// keys_out may be null (last pass: values only).  With sums the workgroups
// also clear the sum rows of multi-piece segments.
__global__ __launch_bounds__(kBlock) void k_digit_scatter(
    const int32_t* __restrict__ keys, const int32_t* __restrict__ vals, int64_t in_stride,
    int64_t N, int64_t K, int first, const int32_t* __restrict__ nvalid, int shift,
    const int32_t* __restrict__ dth, int64_t T, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ vals_out, int64_t out_stride, const int32_t* __restrict__ counts,
    float* __restrict__ sums, int32_t* __restrict__ arrive, int64_t d) {
    __shared__ int32_t s_base[kDigits];
    __shared__ uint32_t s_cur[2][kDigits];
    const int64_t b = blockIdx.y, t = blockIdx.x;
    if (sums) clear_multi_rows(counts + b * K, sums + b * K * d, arrive + b * K, K, d, t, T);
    s_base[threadIdx.x] = dth[(b * T + t) * kDigits + threadIdx.x];
    s_cur[0][threadIdx.x] = 0u;
    s_cur[1][threadIdx.x] = 0u;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n = first ? N : nvalid[b];
    const int64_t w0 = t * kSortTile + (int64_t)wave * kWaveRange;
    const int64_t i1 = min(t * kSortTile + (int64_t)kSortTile, n);
    const int32_t* kin = keys + b * in_stride;
    const int32_t* vin = vals ? vals + b * in_stride : nullptr;
    int32_t* kout = keys_out ? keys_out + b * out_stride : nullptr;
    int32_t* vout = vals_out + b * out_stride;
    uint32_t* cur = s_cur[wave >> 1];
    const uint32_t sh = 16u * (uint32_t)(wave & 1);
    int32_t a[kSortPer], v[kSortPer];
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        const int64_t i = w0 + j * kWave + lane;
        a[j] = i < i1 ? kin[i] : -1;
        v[j] = vin ? (i < i1 ? vin[i] : 0) : (int32_t)i;
    }
#pragma unroll
    for (int j = 0; j < kSortPer; ++j)
        if (a[j] >= 0 && a[j] < K) atomicAdd(&cur[(a[j] >> shift) & (kDigits - 1)], 1u << sh);
    __syncthreads();
    {
        const uint32_t c01 = s_cur[0][threadIdx.x], c23 = s_cur[1][threadIdx.x];
        const uint32_t p1 = c01 & 0xffffu, p2 = p1 + (c01 >> 16), p3 = p2 + (c23 & 0xffffu);
        s_cur[0][threadIdx.x] = p1 << 16;
        s_cur[1][threadIdx.x] = p2 | (p3 << 16);
    }
    __syncthreads();
    const uint64_t below = lane ? ~0ull >> (64 - lane) : 0ull;
#pragma unroll
    for (int j = 0; j < kSortPer; ++j) {
        const bool valid = a[j] >= 0 && a[j] < K;
        const int32_t dig = (a[j] >> shift) & (kDigits - 1);
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (dig >> bit) & 1;
            const uint64_t m = __ballot(on);
            peers &= on ? m : ~m;
        }
        if (!valid) peers = 0;
        const int rank = __popcll(peers & below);
        uint32_t old = 0;
        if (valid && rank == 0) old = atomicAdd(&cur[dig], (uint32_t)__popcll(peers) << sh);
        old = __shfl(old, valid ? __ffsll((unsigned long long)peers) - 1 : lane);
        if (valid) {
            const int32_t pos = s_base[dig] + (int32_t)((old >> sh) & 0xffffu) + rank;
            if (kout) kout[pos] = a[j];
            vout[pos] = v[j];
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

// The same through a buffer resource: the row's byte offset is wave-uniform
// and goes in the scalar offset, the lane's part of the row in the vector
// offset, so a row load costs no vector address arithmetic.  Needs the
// problem's rows to span less than 2 GiB and whole EPL parts (d % EPL == 0).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename T, int EPL>
__device__ inline RowPart<T, EPL> load_row_part_buf(__amdgpu_buffer_rsrc_t rsrc, int32_t row_off,
                                                    int32_t lane_off) {
    constexpr int BYTES = EPL * (int)sizeof(T);
    RowPart<T, EPL> r;
    if constexpr (BYTES == 2) {
        const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(rsrc, lane_off, row_off, 0);
        __builtin_memcpy(r.v, &v, 2);
    } else if constexpr (BYTES == 4) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_off, row_off, 0);
        __builtin_memcpy(r.v, &v, 4);
    } else if constexpr (BYTES == 8) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, lane_off, row_off, 0);
        __builtin_memcpy(r.v, &v, 8);
    } else {
        static_assert(BYTES % 16 == 0, "row part of 16-byte chunks");
        u32x4_t v[BYTES / 16];
#pragma unroll
        for (int c = 0; c < BYTES / 16; ++c)
            v[c] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + 16 * c, row_off, 0);
        __builtin_memcpy(r.v, v, BYTES);
    }
    return r;
}

// Rows gathered per batch: at most 32, and at most 128 VGPRs of row data.
// A piece is a chain of dependent loads (piece table, offsets, indices,
// rows, previous centroid), so waves per SIMD matter as much as rows in
// flight per wave: for 256-byte rows, 64 rows per batch left three waves per
// SIMD and 32 rows leave five (9 % faster at d = 128 fp16 with 64 points per
// cluster, 15-35 % faster with fewer).  Long rows want the opposite: at
// d = 1024 bf16 (about 16 points per cluster) 16 rows per batch at two
// waves per SIMD beat 8 rows at four by 32 %.
template <typename T, int EPL>
constexpr int seg_batch() {
    constexpr int regs = (EPL * (int)sizeof(T) + 3) / 4;
    return regs >= 128 ? 1 : (128 / regs < 32 ? 128 / regs : 32);
}

// Where the segment sums go.  FINAL: the fused finalize writes the new
// centroids (sums and arrive must be zero on entry).  Otherwise partial sums
// are only added into sums (chunks of a streamed pass).
template <typename T>
struct SegOut {
    float* sums;           // [B][K][d]
    int32_t* arrive;       // [B][K]   FINAL
    const float* C_prev;   // [B][K][d] FINAL
    float* C_next;         // [B][K][d] FINAL
    T* lowp;               // [B][K][d] or null
    float* bias;           // [B][K] or null
    uint32_t* move;        // max squared move (fp32 bits) or null
    float* psums;          // [B][M][d] partial sums of pieces, or null (FINAL)
};

// Finalizes centroid row k of problem b from the lane's EPL sums.  EARLY:
// prev already holds the lane's elements of the previous centroid.
template <typename T, int EPL, bool VEC, bool EARLY>
__device__ inline void finalize_row(const SegOut<T>& o, int64_t b, int64_t K, int d, int64_t k,
                                    int32_t count, const float (&s)[EPL], int e0,
                                    const float (&prev)[EPL]) {
    const int64_t base = (b * K + k) * d;
    if (!o.C_next) {
        // sums mode: the segment's sum row itself
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            if (e0 + e < d) o.sums[base + e0 + e] = s[e];
        return;
    }
    const float fn = (float)count;
    float cn = 0.f, mv = 0.f;
    // the previous centroid is read only for the move (C_prev may alias
    // C_next, so before the store)
    const bool want_move = o.move != nullptr;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int j = e0 + e;
        if (j < d) {
            const float c = s[e] / fn;
            const float pv = EARLY ? prev[e] : (want_move ? o.C_prev[base + j] : c);
            o.C_next[base + j] = c;
            float cq = c;
            if (o.lowp) {
                const T q = (T)c;
                o.lowp[base + j] = q;
                cq = to_f32(q);
            }
            cn = fmaf(cq, cq, cn);
            const float m = c - pv;
            mv = fmaf(m, m, mv);
        }
    }
    if (o.bias) {
        cn = wave_sum(cn);
        if ((threadIdx.x & 63) == 0) o.bias[b * K + k] = -0.5f * cn;
    }
    if (o.move) {
        mv = wave_sum(mv);
        if ((threadIdx.x & 63) == 0) atomicMax(o.move, __float_as_uint(mv));
    }
}

// One wave reduces one piece: at most kSegRun consecutive sorted positions
// of a single segment, so the row loop has no boundary to test.  Row indices
// arrive with coalesced loads (one per lane) and are read lane by lane
// (readlane); a batch of RB rows is loaded back to back, then added in
// order.  A segment of one piece is finalized from registers; otherwise the
// piece adds its sums with one row of fp32 atomics, and with FINAL the last
// piece to arrive finalizes the segment.  Extra workgroups past the pieces
// (FINAL only) give empty segments their previous centroid.
// LD = 2: rows load through a buffer resource (d % EPL == 0 and the
// problem's rows span less than 2 GiB); LD = 1: whole parts with 64-bit
// addresses (d % EPL == 0); LD = 0: element by element with bounds.
template <typename T, int EPL, int LD, bool FINAL>
__global__ __launch_bounds__(kBlock) void k_segment_sums(
    const T* __restrict__ X, const int32_t* __restrict__ sorted_idx,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ pieces, SegOut<T> o,
    int64_t N, int64_t K, int d, int64_t M, int64_t piece_wgs) {
    constexpr bool VEC = LD != 0;
    constexpr int RB = seg_batch<T, EPL>();
    constexpr int NV = kSegRun / kWave;  // index registers per lane
    static_assert(kSegRun % RB == 0, "batches tile a piece exactly");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t b = blockIdx.y;
    const int32_t* __restrict__ off = offsets + b * (K + 1);
    const int e0 = lane * EPL;
    const bool active = e0 < d;

    if ((int64_t)blockIdx.x >= piece_wgs) {
        // empty segments keep the previous centroid (FINAL only): a wave
        // checks 64 consecutive segments with one coalesced read of the
        // offsets, then handles the empty ones (usually none) in turn
        if constexpr (FINAL) {
            const int64_t k0 =
                (((int64_t)blockIdx.x - piece_wgs) * (kBlock / kWave) + wave) * kWave;
            const int64_t kl = k0 + lane;
            uint64_t m = __ballot(kl < K && off[kl + 1] == off[kl]);
            while (m) {
                const int64_t k = k0 + __ffsll((unsigned long long)m) - 1;
                m &= m - 1;
                const int64_t base = (b * K + k) * d;
                if (!o.C_next) {  // sums mode: an empty segment sums to zero
                    for (int j = lane; j < d; j += kWave) o.sums[base + j] = 0.f;
                    continue;
                }
                float cn = 0.f;
                const int E = row_part(d);
                for (int e = 0; e < E; ++e) {
                    const int j = lane * E + e;
                    if (j >= d) break;
                    const float c = o.C_prev[base + j];
                    o.C_next[base + j] = c;
                    float cq = c;
                    if (o.lowp) {
                        const T q = (T)c;
                        o.lowp[base + j] = q;
                        cq = to_f32(q);
                    }
                    cn = fmaf(cq, cq, cn);
                }
                if (o.bias) {
                    cn = wave_sum(cn);
                    if (lane == 0) o.bias[b * K + k] = -0.5f * cn;
                }
            }
        }
        return;
    }

    const int32_t* __restrict__ P = pieces + b * (2 * M + 1);
    const int64_t j = (int64_t)blockIdx.x * (kBlock / kWave) + wave;
    // Long rows (EARLY): the piece's slot is read without waiting for the
    // piece count (unused slots hold -1), and the indices and previous
    // centroid are requested before the offsets resolve, so a piece costs
    // one dependent round trip less (9 % at d = 1024 bf16 with 16 points
    // per cluster).  With short rows the later, narrower requests measured
    // 2-3 % faster.
    constexpr bool EARLY = EPL * (int)sizeof(T) >= 16;
    if (EARLY ? j >= M : j >= P[0]) return;
    const int32_t k = __builtin_amdgcn_readfirstlane(P[1 + j]);
    const int32_t p0 = __builtin_amdgcn_readfirstlane(P[1 + M + j]);
    if (EARLY && k < 0) return;
    const T* __restrict__ Xb = X + b * N * d;
    __amdgpu_buffer_rsrc_t rsrc;
    if constexpr (LD == 2)
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(Xb), 0,
                                                 (int32_t)(N * d * (int64_t)sizeof(T)), 0x00020000);
    const int32_t rowb = d * (int32_t)sizeof(T);
    const int32_t lane_off = (active ? e0 : 0) * (int32_t)sizeof(T);
    int32_t vidx[NV];
    float prev[EPL];
    int32_t s0, s1;
    int n;  // rows of this piece
    if constexpr (EARLY) {
        // positions past the piece read the index that follows, up to the
        // last sorted one (past it the array holds no point index when
        // labels were skipped); never added
        const int32_t last = __builtin_amdgcn_readfirstlane(off[K]) - 1;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            vidx[v] = sorted_idx[b * N + min(p0 + v * kWave + lane, last)];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            prev[e] = FINAL && o.C_next && o.move && active && (VEC || e0 + e < d)
                          ? o.C_prev[(b * K + k) * d + e0 + e]
                          : 0.f;
        s0 = __builtin_amdgcn_readfirstlane(off[k]);
        s1 = __builtin_amdgcn_readfirstlane(off[k + 1]);
        n = min(kSegRun, s1 - p0);
    } else {
        s0 = __builtin_amdgcn_readfirstlane(off[k]);
        s1 = __builtin_amdgcn_readfirstlane(off[k + 1]);
        n = min(kSegRun, s1 - p0);
#pragma unroll
        for (int v = 0; v < NV; ++v)
            vidx[v] = sorted_idx[b * N + p0 + min(v * kWave + lane, n - 1)];
#pragma unroll
        for (int e = 0; e < EPL; ++e) prev[e] = 0.f;
    }

    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    // batches of RB rows: all loads first, unconditionally, so they are in
    // flight together (positions past n re-read the last row, lanes past d
    // read the row start; neither is ever added)
#pragma unroll
    for (int base = 0; base < kSegRun; base += RB) {
        if (base < n) {
            RowPart<T, EPL> v[RB];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                const int pos = base + u;
                const int32_t row = __builtin_amdgcn_readlane(vidx[pos / kWave], pos % kWave);
                if constexpr (LD == 2)
                    v[u] = load_row_part_buf<T, EPL>(rsrc, row * rowb, lane_off);
                else
                    v[u] = load_row_part<T, EPL, VEC>(Xb, row, d, active ? e0 : 0);
            }
            // every loaded row is consumed on one path (a select keeps the
            // sum of rows past n unchanged), so no load can be sunk below
            // the waits for the others: a last row loaded only on a
            // full-batch branch cost a whole extra round trip per batch
            if (active) {
#pragma unroll
                for (int u = 0; u < RB; ++u) {
                    const bool in = base + u < n;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        const float t = acc[e] + to_f32(v[u].v[e]);
                        acc[e] = in ? t : acc[e];
                    }
                }
            }
        }
    }

    const int32_t count = s1 - s0;
    if (FINAL && count <= kSegRun) {
        finalize_row<T, EPL, VEC, EARLY>(o, b, K, d, k, count, acc, e0, prev);
        return;
    }
    if (FINAL && o.psums) {
        // two-pass mode: the piece's partial sums for k_merge_pieces
        if (active) {
            float* pp = o.psums + (b * M + j) * d + e0;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                if (VEC || e0 + e < d) pp[e] = acc[e];
        }
        return;
    }
    float* dst = o.sums + (b * K + k) * d + e0;
    if constexpr (FINAL) {
        // Returning atomics: once their results are in, the adds are
        // performed at the device coherence point, so the arrival increment
        // below is ordered after them without a cache write-back fence.
        float done = 0.f;
        if (active) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                if (VEC || e0 + e < d) done += atomicAdd(dst + e, acc[e]);
        }
        asm volatile("" ::"v"(done) : "memory");
        const int32_t npieces = (count + kSegRun - 1) / kSegRun;
        int32_t prior = 0;
        if (lane == 0) prior = atomicAdd(o.arrive + b * K + k, 1);
        prior = __builtin_amdgcn_readfirstlane(prior);
        if (prior == npieces - 1) {
            // Every other piece's adds returned before that piece arrived,
            // so they were performed at the coherence point where this
            // piece's adds and the arrival counter live.  The acquire fence
            // (once per segment of several pieces) keeps the loads below
            // from being served by a stale line in this wave's caches.
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            float t[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                t[e] = active && (VEC || e0 + e < d)
                           ? __hip_atomic_load(dst + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
            finalize_row<T, EPL, VEC, EARLY>(o, b, K, d, k, count, t, e0, prev);
        }
    } else if (active) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            if (VEC || e0 + e < d) atomicAdd(dst + e, acc[e]);
    }
}

// ---------------------------------------------------------------------------
// Second pass of the two-pass segment sums: one wave per segment of more
// than one piece adds the pieces' partial sums in piece order (pieces
// poff[k] .. poff[k] + npieces - 1 cover the segment front to back) and
// finalizes the centroid as the fused path does.
template <typename T>
__global__ __launch_bounds__(kBlock) void k_merge_pieces(const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ poff,
                                                         SegOut<T> o, int64_t K, int d, int64_t M) {
    const int lane = threadIdx.x & 63;
    const int64_t b = blockIdx.y;
    const int64_t k = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    if (k >= K) return;
    const int32_t* off = offsets + b * (K + 1);
    const int32_t count = off[k + 1] - off[k];
    if (count <= kSegRun) return;
    const int32_t np = npieces_of(count);
    const int64_t j0 = poff[b * (K + 1) + k];
    const float* ps = o.psums + (b * M + j0) * d;
    const int64_t base = (b * K + k) * d;
    const float fn = (float)count;
    float cn = 0.f, mv = 0.f;
    const int E = row_part(d);
    for (int e = 0; e < E; ++e) {
        const int j = lane * E + e;
        if (j >= d) break;
        float sum = 0.f;
        for (int32_t q = 0; q < np; ++q) sum += ps[(int64_t)q * d + j];
        if (!o.C_next) {  // sums mode
            o.sums[base + j] = sum;
            continue;
        }
        const float c = sum / fn;
        const float prev = o.C_prev[base + j];
        o.C_next[base + j] = c;
        float cq = c;
        if (o.lowp) {
            const T q = (T)c;
            o.lowp[base + j] = q;
            cq = to_f32(q);
        }
        cn = fmaf(cq, cq, cn);
        const float m = c - prev;
        mv = fmaf(m, m, mv);
    }
    if (!o.C_next) return;
    if (o.bias) {
        cn = wave_sum(cn);
        if (lane == 0) o.bias[b * K + k] = -0.5f * cn;
    }
    if (o.move) {
        mv = wave_sum(mv);
        if (lane == 0) atomicMax(o.move, __float_as_uint(mv));
    }
}

// ---------------------------------------------------------------------------
// Finalize of accumulated sums (streamed path): C_next = sums / counts (or
// C_prev when empty), optional low-precision copy and its bias, squared move
// maximum; clears the sums.
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
    const int E = row_part(d);
    for (int e = 0; e < E; ++e) {
        const int j = lane * E + e;
        if (j >= d) break;
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
hipError_t segment_sums_t(const void* X, const int32_t* sorted_idx, const int32_t* offsets,
                          const int32_t* pieces, const SegParams& sp, int64_t B, int64_t N,
                          int64_t K, int d, hipStream_t s) {
    const int epl = (d + kWave - 1) / kWave;
    const int64_t M = piece_capacity(N, K);
    const int64_t piece_wgs = (M + (kBlock / kWave) - 1) / (kBlock / kWave);
    const int64_t row_wgs = sp.final ? (K + kBlock - 1) / kBlock : 0;  // 64 segments per wave
    const dim3 grid((unsigned)(piece_wgs + row_wgs), (unsigned)B);
    SegOut<T> o{sp.sums, sp.arrive, sp.C_prev, sp.C_next, static_cast<T*>(sp.lowp), sp.bias,
                sp.move, sp.final ? sp.psums : nullptr};
    const T* x = static_cast<const T*>(X);
    auto merge = [&](hipError_t e) {
        if (e != hipSuccess || !o.psums) return e;
        const dim3 mgrid((unsigned)((K + (kBlock / kWave) - 1) / (kBlock / kWave)), (unsigned)B);
        hipLaunchKernelGGL((k_merge_pieces<T>), mgrid, dim3(kBlock), 0, s, offsets, sp.poff, o,
                           K, d, M);
        return hipGetLastError();
    };
#define FK_SEG_LAUNCH(E, V, F)                                                                 \
    hipLaunchKernelGGL((k_segment_sums<T, E, V, F>), grid, dim3(kBlock), 0, s, x, sorted_idx,  \
                       offsets, pieces, o, N, K, d, M, piece_wgs)
    // buffer loads need whole parts and rows spanning less than 2 GiB per problem
    const bool buf_ok = N * (int64_t)d * (int64_t)sizeof(T) < ((int64_t)1 << 31);
#define FK_SEG_CASE(E)                                                                         \
    if (epl <= E) {                                                                            \
        const int ld = d % E != 0 ? 0 : (buf_ok ? 2 : 1);                                      \
        if (sp.final) {                                                                        \
            if (ld == 2) FK_SEG_LAUNCH(E, 2, true);                                            \
            else if (ld == 1) FK_SEG_LAUNCH(E, 1, true);                                       \
            else FK_SEG_LAUNCH(E, 0, true);                                                    \
        } else {                                                                               \
            if (ld == 2) FK_SEG_LAUNCH(E, 2, false);                                           \
            else if (ld == 1) FK_SEG_LAUNCH(E, 1, false);                                      \
            else FK_SEG_LAUNCH(E, 0, false);                                                   \
        }                                                                                      \
        return merge(hipGetLastError());                                                       \
    }
    FK_SEG_CASE(1)
    FK_SEG_CASE(2)
    FK_SEG_CASE(4)
    FK_SEG_CASE(8)
    FK_SEG_CASE(16)
#undef FK_SEG_CASE
#undef FK_SEG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace

// ---------------------------------------------------------------------------
bool sort_tiled(int64_t N, int64_t K) {
    const int64_t T = (N + kSortTile - 1) / kSortTile;
    return K <= kTiledBinsMax && T * (K + 1) <= 4 * N + 65536;
}

int64_t sort_table_bound(int64_t N, int64_t K) {
    const int64_t T = (N + kSortTile - 1) / kSortTile;
    if (sort_tiled(N, K)) return T * (K + 1);
    return T * kDigits;  // radix passes: per-tile digit counts
}

int64_t radix_pairs_bound(int64_t N, int64_t K) { return sort_tiled(N, K) ? 0 : 4 * N; }

int radix_passes(int64_t K) {
    int bits = 0;
    while (bits < 31 && ((int64_t)1 << bits) < K) ++bits;  // labels < 2^bits
    return bits <= 8 ? 1 : (bits + 7) / 8;
}

hipError_t launch_fill_u32(uint32_t* ptr, int64_t n, uint32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = min((n + kBlock - 1) / kBlock, (int64_t)4096);
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(kBlock), 0, s, ptr, n, value);
    return hipGetLastError();
}

hipError_t launch_add_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = min((n + kBlock - 1) / kBlock, (int64_t)4096);
    hipLaunchKernelGGL(k_add_f32, dim3((unsigned)blocks), dim3(kBlock), 0, s, dst, src, n);
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

hipError_t launch_sort(const SortParams& sp, int64_t B, int64_t N, int64_t K, hipStream_t s) {
    const int64_t T = (N + kSortTile - 1) / kSortTile;
    const int64_t M = piece_capacity(N, K);
    const dim3 tiles((unsigned)T, (unsigned)B);
    const bool tiled = sort_tiled(N, K);
    const int use_lds = K <= kLdsBinsMax;
    const size_t lds = use_lds ? (size_t)K * sizeof(int32_t) : 0;
    if (tiled) {
        hipLaunchKernelGGL(k_tile_hist, tiles, dim3(kBlock), (size_t)(K + 1) * sizeof(int32_t), s,
                           sp.labels, sp.table, N, K, T);
        const dim3 cgrid((unsigned)((K + kWave) / kWave), (unsigned)B);
        if (T >= 64)
            hipLaunchKernelGGL(k_tile_colscan<16>, cgrid, dim3(16 * kWave), 0, s, sp.table,
                               sp.counts, sp.bad, K, T);
        else
            hipLaunchKernelGGL(k_tile_colscan<4>, cgrid, dim3(4 * kWave), 0, s, sp.table,
                               sp.counts, sp.bad, K, T);
    } else {
        ZeroRanges z{};
        z.p[0] = reinterpret_cast<uint32_t*>(sp.counts);
        z.n[0] = B * K;
        z.p[1] = reinterpret_cast<uint32_t*>(sp.bad);
        z.n[1] = B;
        const int64_t zb = min((B * K + kBlock - 1) / kBlock, (int64_t)4096);
        hipLaunchKernelGGL(k_zero, dim3((unsigned)zb), dim3(kBlock), 0, s, z);
        hipLaunchKernelGGL(k_histogram, tiles, dim3(kBlock), lds, s, sp.labels, sp.counts, sp.bad,
                           N, K, use_lds);
    }
    const int64_t nblk = (K + kPlanBlock - 1) / kPlanBlock;
    if (nblk > 1)
        hipLaunchKernelGGL(k_plan_totals, dim3((unsigned)nblk, (unsigned)B), dim3(kBlock), 0, s,
                           sp.counts, sp.part, K);
    hipLaunchKernelGGL(k_plan, dim3((unsigned)nblk, (unsigned)B), dim3(kPlanThreads), 0, s, sp.counts,
                       sp.part, sp.offsets, sp.poff, sp.pieces, sp.move, K, M);
    if (tiled) {
        // consecutive tiles per XCD (scatter_tile) whenever the 1-D grid fits
        // (nothing to merge when every problem is one tile)
        const int64_t pairs = T > 1 && 8 * ((T * B + 7) / 8) < ((int64_t)1 << 31) ? T * B : 0;
        const dim3 sgrid = pairs ? dim3((unsigned)(8 * ((pairs + 7) / 8))) : tiles;
        const int nbits = K > 1 ? 64 - __builtin_clzll((unsigned long long)(K - 1)) : 0;
        if (K <= kWaveBinsMax) {
            constexpr int NW = kScatterWaves;
            static LdsAttr attr;
            const hipError_t e = ensure_lds(attr, reinterpret_cast<const void*>(k_tile_scatter_w<NW>),
                                            scatter_w_lds<NW>(kWaveBinsMax));
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(k_tile_scatter_w<NW>, sgrid, dim3(NW * kWave),
                               (size_t)scatter_w_lds<NW>(K), s, sp.labels, sp.table, sp.offsets,
                               sp.sorted_idx, sp.counts, sp.sums, sp.arrive, N, K, T, sp.d,
                               pairs, nbits);
        } else
            hipLaunchKernelGGL(k_tile_scatter, sgrid, dim3(kBlock), (size_t)K * sizeof(int32_t), s,
                               sp.labels, sp.table, sp.offsets, sp.sorted_idx, sp.counts, sp.sums,
                               sp.arrive, N, K, T, sp.d, pairs, nbits);
    } else {
        // LSD radix passes over 8-bit digits; pairs ping-pong between the
        // two halves of the radix buffer, the last pass writes sorted_idx
        const int np = radix_passes(K);
        const int64_t RP = radix_pairs_bound(N, K);
        for (int q = 0; q < np; ++q) {
            const bool first = q == 0, last = q == np - 1;
            const int32_t* kin = first ? sp.labels : sp.radix + ((q - 1) % 2) * 2 * N;
            const int32_t* vin = first ? nullptr : kin + N;
            const int64_t in_stride = first ? N : RP;
            int32_t* kout = last ? nullptr : sp.radix + (q % 2) * 2 * N;
            int32_t* vout = last ? sp.sorted_idx : kout + N;
            const int64_t out_stride = last ? N : RP;
            hipLaunchKernelGGL(k_digit_hist, tiles, dim3(kBlock), 0, s, kin, in_stride, N, K,
                               (int)first, sp.nvalid, 8 * q, sp.table, T);
            hipLaunchKernelGGL(k_digit_colscan, dim3((unsigned)B), dim3(kDigits * kDigitGroups),
                               0, s, sp.table, sp.nvalid, T);
            hipLaunchKernelGGL(k_digit_scatter, tiles, dim3(kBlock), 0, s, kin, vin, in_stride, N,
                               K, (int)first, sp.nvalid, 8 * q, sp.table, T, kout, vout,
                               out_stride, sp.counts, last ? sp.sums : nullptr, sp.arrive, sp.d);
        }
    }
    return hipGetLastError();
}

hipError_t launch_segment_sums(int dtype, const void* X, const int32_t* sorted_idx,
                               const int32_t* offsets, const int32_t* pieces,
                               const SegParams& sp, int64_t B, int64_t N, int64_t K, int d,
                               hipStream_t s) {
    switch (dtype) {
        case FK_F32:
            return segment_sums_t<float>(X, sorted_idx, offsets, pieces, sp, B, N, K, d, s);
        case FK_F16:
            return segment_sums_t<_Float16>(X, sorted_idx, offsets, pieces, sp, B, N, K, d, s);
        default:
            return segment_sums_t<__bf16>(X, sorted_idx, offsets, pieces, sp, B, N, K, d, s);
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
