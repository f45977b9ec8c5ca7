/*
 * fk_baseline.h -- the unfused forms of the two Lloyd stages, exported by the
 * same library as fk.h for comparison on the same hardware.  They are not
 * used by any fk.h entry point.
 *
 * The notes the library follows (papernotes.org, "Flash-KMeans: Fast and
 * Memory-Efficient Exact K-Means", 核心问题) name two bottlenecks of a
 * straightforward Lloyd iteration on a GPU:
 *   - the assignment writes the whole N x K distance matrix to device memory
 *     and reads it back for the argmin (IO of order NK rather than Nd + Kd);
 *   - the update adds every point into its centroid's sum with atomic adds,
 *     which serialise on centroids that many points share.
 * fk_baseline_scores + fk_baseline_argmin form the first, the
 * materialised-matrix assignment; fk_baseline_update_scatter is the second,
 * the scatter-atomic update.  Their results are those of fk_assign and
 * fk_update (same labels on the same scores; same counts, centroids up to the
 * order of the fp32 additions).
 *
 * Conventions (shapes, dtypes, ties, memory, streams, errors) are those of
 * fk.h.  None of these calls takes a workspace: the buffers they write are
 * arguments.
 */
#ifndef FK_BASELINE_H
#define FK_BASELINE_H

#include "fk.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fk_baseline_scores -- the score matrix of the distance expansion
 * (papernotes.org notes, 关键设计 1: |x - c|^2 = |x|^2 + |c|^2 - 2 x.c, with
 * |x|^2 constant per point): D[b][i][k] = x_bi . c_bk + bias[b][k] in fp32,
 * the dot product accumulated in fp32 from the stored 16-bit values by the
 * same matrix-instruction tiles as fk_assign.  bias [B][K] fp32 as written
 * by fk_centroid_bias.  D [B][N][K] fp32 (B*N*K*4 bytes), written entirely.
 * fp16 and bf16 problems with d <= 256 only (FK_EUNSUPPORTED otherwise).
 */
fk_status fk_baseline_scores(const fk_problem* p, const void* X, const void* C, const float* bias,
                             float* D, void* stream);

/*
 * fk_baseline_argmin -- labels[b][i] = the lowest k among the largest of
 * D[b][i][0..K) (the nearest centroid: larger score, smaller distance).
 * D [B][N][K] fp32, labels [B][N] int32.
 */
fk_status fk_baseline_argmin(const fk_problem* p, const float* D, int32_t* labels, void* stream);

/*
 * fk_baseline_update_scatter -- the update by atomics (papernotes.org notes,
 * 核心问题, the contended form): sums[b][a][j] += X[b][i][j] with one fp32
 * atomic add per element and counts[b][a] += 1 per point, a = labels[b][i];
 * then C_next = sums / counts in fp32, or C_prev when a count is 0.
 *   X, labels, C_prev, C_next, C_next_lowp, counts as in fk_update
 *     (C_prev may alias C_next);
 *   sums [B][K][d] fp32 scratch, cleared on entry and left zero.
 * Labels outside [0, K) are skipped (not counted by fk_error_count).  The
 * centroid low bits depend on the order of the atomic additions.
 */
fk_status fk_baseline_update_scatter(const fk_problem* p, const void* X, const int32_t* labels,
                                     const float* C_prev, float* C_next, void* C_next_lowp,
                                     int32_t* counts, float* sums, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FK_BASELINE_H */
