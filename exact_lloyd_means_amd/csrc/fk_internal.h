// fk_internal.h -- declarations shared by the library's translation units:
// device vector types, the workspace layout and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fk.h"
#include "../../include/fk_baseline.h"
#include "../../include/fk_tune.h"

#include <atomic>

namespace fk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Element size in bytes of a problem dtype.
inline int dtype_size(int dtype) { return dtype == FK_F32 ? 4 : 2; }

// Most sorted positions one wave reduces in the segment-sum kernel (a piece:
// part of a single segment).
constexpr int kSegRun = 256;
// Pieces a problem can have: sum over segments of ceil(count / kSegRun).
inline int64_t piece_capacity(int64_t N, int64_t K) { return (N + kSegRun - 1) / kSegRun + K; }
// Labels per workgroup of the plan (offsets and pieces) and blocks per problem.
constexpr int64_t kPlanLabels = 4096;
inline int64_t plan_blocks(int64_t K) { return (K + kPlanLabels - 1) / kPlanLabels; }

// Counting sort plan: the tiled form (per-tile count table, no global
// atomics) when K is small enough for LDS bins and the table stays modest.
bool sort_tiled(int64_t N, int64_t K);
// int32 entries per problem of the sort table (tile table or cursors), an
// upper bound for every N' <= N
int64_t sort_table_bound(int64_t N, int64_t K);

// int32 entries per problem of the radix sort's (label, point) pair buffers
// (0 when the tiled sort applies)
int64_t radix_pairs_bound(int64_t N, int64_t K);

// Workspace layout.  Every region starts on a 256-byte boundary.  Sizes grow
// with B*K*d, B*N and B*K only: the N x K distance matrix has no place here.
struct Workspace {
    float* bias;         // [B][K]   -0.5 |c|^2 of the centroids an assign reads
    int32_t* offsets;    // [B][K+1] segment starts of the sorted labels
    int32_t* table;      // [B][sort_table_bound] per-tile label or digit counts
    int32_t* radix;      // [B][radix_pairs_bound] pair buffers of the radix sort
    int32_t* nvalid;     // [B]      valid labels (radix sort)
    int32_t* sorted_idx; // [B][N]   argsort of the labels
    int32_t* poff;       // [B][K+1] first piece of each segment
    int32_t* pieces;     // [B][1 + 2 * piece_capacity] piece count, segments, starts
    int32_t* part;       // [B][2 * plan_blocks(K)] block totals of the plan
    float* sums;         // [B][K][d] fp32 segment sums
    int32_t* arrive;     // [B][K]   pieces of each segment added so far
    int32_t* counts;     // [B][K]   counts when the caller passes none
    void* lowp;          // [B][K][d] centroids in the problem dtype (16-bit dtypes)
    int32_t* bad;        // [B]      labels outside [0, K) per problem
    uint32_t* flags;     // [1] max squared move (fp32 bits)
    float* psums;        // [B][piece_capacity][d] piece partial sums (FK_DETERMINISTIC), or null
    size_t total;
};

Workspace workspace_layout(const fk_problem& p, char* base);

// Workspace of the streamed path: two chunk buffers of X, the sort scratch
// of one chunk, and the per-problem sums, bias and low-precision centroids.
struct StreamWorkspace {
    void* xbuf[2];       // [chunk][d] problem dtype
    float* bias;         // [B][K]
    void* lowp;          // [B][K][d] (16-bit dtypes)
    float* sums;         // [B][K][d]
    int32_t* ccounts;    // [K]   counts of one chunk
    int32_t* offsets;    // [K+1] segment starts of one chunk
    int32_t* table;      // [sort_table_bound(chunk)]
    int32_t* radix;      // [radix_pairs_bound(chunk)]
    int32_t* nvalid;     // [1]
    int32_t* sorted_idx; // [chunk]
    int32_t* poff;       // [K+1]
    int32_t* pieces;     // [1 + 2 * piece_capacity(chunk)]
    int32_t* part;       // [2 * plan_blocks(K)]
    int32_t* bad;        // [1]
    float* csums;        // [K][d] one chunk's segment sums (FK_DETERMINISTIC), or null
    float* psums;        // [piece_capacity(chunk)][d] piece partials (FK_DETERMINISTIC), or null
    size_t total;
};

StreamWorkspace stream_workspace_layout(const fk_problem& p, int64_t chunk, char* base);

// Argument block of the counting sort.
struct SortParams {
    const int32_t* labels;  // [B][N]
    int32_t* counts;        // [B][K]
    int32_t* offsets;       // [B][K+1]
    int32_t* sorted_idx;    // [B][N]
    int32_t* poff;          // [B][K+1]
    int32_t* pieces;        // [B][1 + 2 * piece_capacity]
    int32_t* table;         // [B][sort_table_bound]
    int32_t* radix;         // [B][radix_pairs_bound] (radix sort only)
    int32_t* nvalid;        // [B] (radix sort only)
    int32_t* bad;           // [B]
    uint32_t* move;         // cleared when not null
    float* sums;            // [B][K][d] rows of multi-piece segments cleared (or null)
    int32_t* arrive;        // [B][K]   their arrival counters cleared
    int32_t* part;          // [B][2 * plan_blocks(K)] block totals of the plan
    int64_t d;
};

// Argument block of the segment sums.  final: fused finalize into C_next
// (sums and arrive must be zero), or, with C_next null, every segment's sum
// row stored into sums (sums mode, zero rows for empty segments); otherwise
// partial sums are added to sums.
struct SegParams {
    bool final;
    float* sums;
    int32_t* arrive;
    const float* C_prev;
    float* C_next;
    void* lowp;       // problem dtype, or null
    float* bias;      // or null
    uint32_t* move;   // or null
    // final only: when set, the pieces of multi-piece segments store their
    // partial sums here ([B][piece_capacity][d] fp32) instead of adding them
    // with atomics, and a second pass adds them in piece order (a result
    // that does not depend on timing); poff [B][K+1] = first piece of each
    // segment
    float* psums;
    const int32_t* poff;
};

// Raises a kernel's dynamic LDS limit to `bytes` once per device (the
// attribute is a property of the function on the current device).  `rec` is
// the kernel's own record: one bit per device ordinal below 64 (others set
// the attribute on every launch).
struct LdsAttr {
    std::atomic<uint64_t> done{0};
};
inline hipError_t ensure_lds(LdsAttr& rec, const void* kern, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (rec.done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) rec.done.fetch_or(bit, std::memory_order_release);
    return e;
}

// ---- launchers (return hipSuccess or the launch error) ----------------------
hipError_t launch_fill_u32(uint32_t* ptr, int64_t n, uint32_t value, hipStream_t s);

// dst[i] += src[i]
hipError_t launch_add_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s);
hipError_t launch_add_f32(float* dst, const float* src, int64_t n, hipStream_t s);

hipError_t launch_centroid_bias(int dtype, const void* C, float* bias, int64_t rows, int d,
                                hipStream_t s);

// Round fp32 centroids to the problem dtype (16-bit only) and compute the bias
// of the rounded values.
hipError_t launch_prepare(int dtype, const float* C, void* lowp, float* bias, int64_t rows, int d,
                          hipStream_t s);

hipError_t launch_assign(int dtype, const void* X, const void* C, const float* bias,
                         int32_t* labels, float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                         hipStream_t s);

hipError_t launch_sort(const SortParams& sp, int64_t B, int64_t N, int64_t K, hipStream_t s);

hipError_t launch_segment_sums(int dtype, const void* X, const int32_t* sorted_idx,
                               const int32_t* offsets, const int32_t* pieces,
                               const SegParams& sp, int64_t B, int64_t N, int64_t K, int d,
                               hipStream_t s);

// C_next = sums / counts (or C_prev when empty); optional low-precision copy,
// bias of the copy, squared-move maximum; clears the sums.
hipError_t launch_finalize(int dtype, float* sums, const int32_t* counts, const float* C_prev,
                           float* C_next, void* lowp, float* bias, uint32_t* move_max,
                           int64_t rows, int d, hipStream_t s);

// fp16 fused assign with an explicit shape (d = 64, 128 or 256)
hipError_t launch_assign_variant(const void* X, const void* C, const float* bias, int32_t* labels,
                                 int64_t B, int64_t N, int64_t K, int d, int np, int waves,
                                 int64_t grid_wgs, hipStream_t s);

// ---- baselines: materialised scores + argmin, scatter-atomic update --------
// D [B][N][K] fp32 = x.c + bias for 16-bit inputs with d <= 256.
hipError_t launch_scores(int dtype, const void* X, const void* C, const float* bias, float* D,
                         int64_t B, int64_t N, int64_t K, int d, hipStream_t s);

// labels[r] = lowest index of the largest of D[r][0..K)
hipError_t launch_argmin_rows(const float* D, int32_t* labels, int64_t rows, int64_t K,
                              hipStream_t s);

// sums[b][labels[b][i]] += X[b][i] and counts[b][labels[b][i]] += 1 with atomics
hipError_t launch_scatter_add(int dtype, const void* X, const int32_t* labels, float* sums,
                              int32_t* counts, int64_t B, int64_t N, int64_t K, int d,
                              hipStream_t s);

}  // namespace fk
