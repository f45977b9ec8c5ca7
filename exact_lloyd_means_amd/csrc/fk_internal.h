// fk_internal.h -- declarations shared by the library's translation units:
// device vector types, the workspace layout and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fk.h"

namespace fk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Element size in bytes of a problem dtype.
inline int dtype_size(int dtype) { return dtype == FK_F32 ? 4 : 2; }

// Workspace layout.  Every region starts on a 256-byte boundary.  Sizes grow
// with B*K*d, B*N and B*K only: the N x K distance matrix has no place here.
struct Workspace {
    float* bias;         // [B][K]   -0.5 |c|^2 of the centroids an assign reads
    int32_t* offsets;    // [B][K+1] segment starts of the sorted labels
    int32_t* cursor;     // [B][K]   scatter cursors
    int32_t* sorted_idx; // [B][N]   argsort of the labels
    int32_t* sorted_lab; // [B][N]   label at each sorted position
    float* sums;         // [B][K][d] fp32 segment sums
    int32_t* counts;     // [B][K]   counts when the caller passes none
    void* lowp;          // [B][K][d] centroids in the problem dtype (16-bit dtypes)
    uint32_t* flags;     // [0] out-of-range labels, [1] max squared move (fp32 bits)
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
    int32_t* cursor;     // [K]
    int32_t* sorted_idx; // [chunk]
    int32_t* sorted_lab; // [chunk]
    uint32_t* flags;     // [0] out-of-range labels
    size_t total;
};

StreamWorkspace stream_workspace_layout(const fk_problem& p, int64_t chunk, char* base);

// ---- launchers (return hipSuccess or the launch error) ----------------------
hipError_t launch_fill_u32(uint32_t* ptr, int64_t n, uint32_t value, hipStream_t s);

// dst[i] += src[i]
hipError_t launch_add_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s);

hipError_t launch_centroid_bias(int dtype, const void* C, float* bias, int64_t rows, int d,
                                hipStream_t s);

// Round fp32 centroids to the problem dtype (16-bit only) and compute the bias
// of the rounded values.
hipError_t launch_prepare(int dtype, const float* C, void* lowp, float* bias, int64_t rows, int d,
                          hipStream_t s);

hipError_t launch_assign(int dtype, const void* X, const void* C, const float* bias,
                         int32_t* labels, float* min_dist, int64_t B, int64_t N, int64_t K, int d,
                         hipStream_t s);

hipError_t launch_histogram(const int32_t* labels, int32_t* counts, uint32_t* flags, int64_t B,
                            int64_t N, int64_t K, hipStream_t s);

hipError_t launch_scan(const int32_t* counts, int32_t* offsets, int32_t* cursor, int64_t B,
                       int64_t K, hipStream_t s);

// sorted_lab may be NULL
hipError_t launch_scatter(const int32_t* labels, int32_t* cursor, int32_t* sorted_idx,
                          int32_t* sorted_lab, int64_t B, int64_t N, int64_t K, hipStream_t s);

hipError_t launch_segment_sums(int dtype, const void* X, const int32_t* sorted_idx,
                               const int32_t* sorted_lab, const int32_t* offsets, float* sums,
                               int64_t B, int64_t N, int64_t K, int d, hipStream_t s);

// C_next = sums / counts (or C_prev when empty); optional low-precision copy,
// bias of the copy, squared-move maximum; clears the sums.
hipError_t launch_finalize(int dtype, float* sums, const int32_t* counts, const float* C_prev,
                           float* C_next, void* lowp, float* bias, uint32_t* move_max,
                           int64_t rows, int d, hipStream_t s);

}  // namespace fk
