/*
 * fk.h -- C ABI of an exact batched Lloyd k-means library for AMD Instinct
 * MI355X (gfx950).
 *
 * One Lloyd iteration has two stages (7minutos.es article on Flash-KMeans,
 * "¿Qué es Flash-KMeans?"; papernotes.org notes "Flash-KMeans: Fast and
 * Memory-Efficient Exact K-Means", 方法详解 / 整体框架):
 *   assign -- every point takes the index of its nearest centroid, found by a
 *             fused distance + running (min, argmin) pass that never stores
 *             the N x K distance matrix (papernotes.org notes, 关键设计 1);
 *   update -- every centroid becomes the mean of its points, computed by
 *             argsorting the labels and reducing contiguous same-label
 *             segments, X never permuted (papernotes.org notes, 关键设计 2).
 * The result equals textbook Lloyd; nothing is approximated.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Shapes   B independent problems with the same N (points), K (centroids)
 *           and d (dimensions).  X is [B][N][d], C is [B][K][d], labels
 *           [B][N], counts [B][K], offsets [B][K+1], all contiguous and
 *           row-major.
 *  Types    X and the centroids an assignment reads are stored in the
 *           problem dtype (fp32, fp16 or bf16).  Dot products accumulate in
 *           fp32.  Centroids carried between iterations, sums and the
 *           centroid bias are fp32.  Labels, counts, offsets and sorted
 *           indices are int32; labels are 0-based, in [0, K).
 *  Ties     Among centroids at exactly equal computed distance the lowest
 *           index wins.
 *  Empty    A centroid with no points keeps its previous value bit for bit.
 *  Memory   Every pointer is a device pointer unless marked "host".  Device
 *           pointers must be 16-byte aligned.  The caller owns every buffer;
 *           the library allocates no device memory, keeps no pointer after a
 *           call returns and holds no state between calls (fk_last_error
 *           aside).  Scratch space comes from the caller's workspace `ws`
 *           of `ws_bytes` bytes (see fk_workspace_size); only
 *           fk_update_bias_noalloc uses the library's static scratch
 *           instead.
 *  Streams  `stream` is a hipStream_t passed as void*; NULL is the null
 *           stream.  All device work is enqueued asynchronously on it.
 *           Calls on different streams are safe when their workspaces and
 *           outputs are distinct.
 *  Errors   Arguments are checked on the host before anything is enqueued;
 *           on an error nothing is enqueued and outputs are untouched.
 *           FK_EINVAL     null required pointer, a size < 1, misalignment;
 *           FK_EUNSUPPORTED unknown dtype or a size beyond the limits below;
 *           FK_EWORKSPACE workspace missing or smaller than required;
 *           FK_EHIP       a HIP runtime call or launch failed;
 *           FK_EHOST      a host-side resource failed (streamed path).
 *           fk_last_error() describes the most recent failure on the
 *           calling thread.  Faults inside kernels surface at the caller's
 *           next synchronisation.
 *  Limits   N, K <= 2^31 - 2; d <= 65536.  Inputs must be finite, and
 *           |c|^2 must be finite in fp32; otherwise labels are undefined
 *           (but stay in [0, K)).  A point with a non-finite coordinate
 *           does not change the labels of the other points.
 */
#ifndef FK_H
#define FK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FK_ABI_VERSION 1

typedef enum fk_dtype { FK_F32 = 0, FK_F16 = 1, FK_BF16 = 2 } fk_dtype;

typedef enum fk_status {
    FK_OK = 0,
    FK_EINVAL = -1,
    FK_EUNSUPPORTED = -2,
    FK_EWORKSPACE = -3,
    FK_EHIP = -4,
    FK_EHOST = -5
} fk_status;

/*
 * Problem flags (fk_problem.flags, bitwise or; other bits must be 0).
 *
 * FK_DETERMINISTIC -- results of fk_update and fk_lloyd do not depend on
 *   timing: the same inputs give the same bits on every run.  (The argsort
 *   is always stable.)  Segments longer than 256 points store each piece's
 *   partial sums (workspace) and add them in piece order in a second pass
 *   instead of with atomics; fk_lloyd_streamed stores each chunk's sums and
 *   adds them to the running sums in chunk order.  The workspace grows by
 *   B * (ceil(N/256) + K) * d * 4 bytes (streamed: (ceil(chunk/256) + 2 K)
 *   * d * 4 bytes).
 */
#define FK_DETERMINISTIC 1

/* Problem description shared by all calls.  dtype is an fk_dtype value;
 * flags a combination of the FK_* flags above (0: none). */
typedef struct fk_problem {
    int64_t B, N, K, d;
    int32_t dtype;
    int32_t flags;
} fk_problem;

/* Version of this ABI (FK_ABI_VERSION of the built library). */
int fk_abi_version(void);

/* Static text for a status code. */
const char* fk_status_str(int status);

/* Text of the most recent error on the calling thread ("" if none). */
const char* fk_last_error(void);

/*
 * fk_workspace_size -- bytes of device workspace the other calls need for
 * problem *p.  chunk_points = 0: fk_assign, fk_sort_labels, fk_update and
 * fk_lloyd; chunk_points > 0: fk_lloyd_streamed with chunks of that many
 * points (capped at N).  The size has no N x K term: the distance matrix is never stored
 * (papernotes.org notes, 关键设计 1: IO falls from O(NK) to O(Nd + Kd)).
 * *bytes (host) receives the size.
 */
fk_status fk_workspace_size(const fk_problem* p, int64_t chunk_points, size_t* bytes);

/*
 * fk_workspace_bytes -- the same size returned directly: bytes of device
 * workspace for problem *p (chunk_points as in fk_workspace_size).  Returns
 * 0 when the problem or chunk_points is invalid; fk_last_error() then says
 * why.  No N x K term, as above.
 */
size_t fk_workspace_bytes(const fk_problem* p, int64_t chunk_points);

/*
 * fk_centroid_bias -- the centroid term of the distance expansion
 * |x - c|^2 = |x|^2 + |c|^2 - 2 x.c (papernotes.org notes, 关键设计 1):
 * bias[b][k] = -0.5 * sum_j C[b][k][j]^2, accumulated in fp32 from the
 * stored dtype values of C [B][K][d].  bias is fp32 [B][K].
 */
fk_status fk_centroid_bias(const fk_problem* p, const void* C, float* bias, void* stream);

/*
 * fk_assign -- nearest centroid of every point (papernotes.org notes,
 * 关键设计 1, running minimum m <- +inf, index a <- -1, merged by min/argmin).
 * X [B][N][d] and C [B][K][d] in the problem dtype.  Writes labels [B][N]
 * (int32, lowest index on exact ties of the fp32 score x.c - |c|^2/2) and,
 * when min_dist is not NULL, min_dist [B][N] = |x|^2 - 2 max_k(x.c - |c|^2/2)
 * in fp32, the squared distance to the chosen centroid.  Uses ws for the
 * centroid bias.  The N x K distance matrix is never written.
 */
fk_status fk_assign(const fk_problem* p, const void* X, const void* C, int32_t* labels,
                    float* min_dist, void* ws, size_t ws_bytes, void* stream);

/*
 * fk_assign_with_bias -- fk_assign with the centroid bias supplied by the
 * caller: bias [B][K] fp32 must equal fk_centroid_bias(C) for the result to
 * be the nearest-centroid assignment.  Needs no workspace.  Lets a caller
 * that keeps C fixed over many assignments (or that gets the bias from
 * fk_lloyd's finalize) skip the bias pass.
 */
fk_status fk_assign_with_bias(const fk_problem* p, const void* X, const void* C,
                              const float* bias, int32_t* labels, float* min_dist, void* stream);

/*
 * fk_sort_labels -- the argsort half of the update (papernotes.org notes,
 * 关键设计 2: the 1-D label vector is argsorted so equal labels form
 * contiguous segments).  From labels [B][N] writes
 *   counts     [B][K]   number of points per label (exact);
 *   offsets    [B][K+1] exclusive prefix sums of counts (offsets[b][K] = the
 *                       number of labels in [0, K), N when all are valid);
 *   sorted_idx [B][N]   point indices grouped by label: positions
 *                       offsets[b][k] .. offsets[b][k+1]-1 hold the points of
 *                       label k, in increasing index order (a stable
 *                       argsort).
 * Labels outside [0, K) are skipped and counted (fk_error_count).
 */
fk_status fk_sort_labels(const fk_problem* p, const int32_t* labels, int32_t* counts,
                         int32_t* offsets, int32_t* sorted_idx, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * fk_update -- new centroids from labels (papernotes.org notes, 关键设计 2):
 * argsort the labels, gather the rows of X of each contiguous same-label
 * segment (X is not moved), sum them in fp32 on chip, then divide by the
 * count.  A segment of at most 256 points is summed by one wave without
 * atomics; a longer one is cut into pieces of 256 sorted positions, each
 * adding its partial sum with one row of fp32 atomic adds.
 *   X [B][N][d] problem dtype; labels [B][N];
 *   C_prev [B][K][d] fp32, kept for empty clusters (may alias C_next);
 *   C_next [B][K][d] fp32 = sum / count (IEEE fp32 division);
 *   C_next_lowp [B][K][d] problem dtype = C_next rounded to nearest even,
 *     may be NULL (must be NULL or distinct from C_next for fp32);
 *   counts [B][K] int32.
 * The fp32 sums follow the sorted order within each segment (increasing
 * point index) and, for segments longer than 256 points, the order of the
 * atomic additions of their pieces, so without FK_DETERMINISTIC the low
 * bits of such centroids can differ between runs; with it they cannot.
 * Counts never differ.  Labels outside [0, K) are skipped and counted
 * (fk_error_count).
 */
fk_status fk_update(const fk_problem* p, const void* X, const int32_t* labels,
                    const float* C_prev, float* C_next, void* C_next_lowp, int32_t* counts,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * fk_update_bias -- fk_update that also writes the centroid bias of the new
 * centroids for the next assignment (the ||c||^2 term of papernotes.org
 * notes, 关键设计 1, computed in the finalize instead of a separate pass):
 * bias_next [B][K] fp32 = -0.5 |c|^2 of C_next_lowp (of C_next for fp32
 * or when C_next_lowp is NULL), bit for bit what fk_centroid_bias would
 * return for those values.  bias_next may be the buffer the assignment
 * that produced labels read (work on one stream runs in order).
 */
fk_status fk_update_bias(const fk_problem* p, const void* X, const int32_t* labels,
                         const float* C_prev, float* C_next, void* C_next_lowp, int32_t* counts,
                         float* bias_next, void* ws, size_t ws_bytes, void* stream);

/*
 * Bytes of the static scratch of fk_update_bias_noalloc, per device.
 */
#define FK_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * fk_update_bias_noalloc -- fk_update_bias for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without ws and
 * ws_bytes, the same kernels and results, and nothing allocated, by the
 * library or by the caller.  Its scratch is one array of
 * FK_NOALLOC_SCRATCH_BYTES bytes in the library's code object: each GPU
 * the library runs on holds its own copy until the process ends.  The
 * first call on a device (the device of `stream`, the current device for
 * the null stream) looks up the array's address there; later calls reuse
 * it.
 *   Size     a problem whose workspace (fk_workspace_size with chunk_points
 *            = 0) exceeds FK_NOALLOC_SCRATCH_BYTES is rejected with
 *            FK_EUNSUPPORTED before anything is enqueued (B = 32, N = 65536,
 *            K = 1024, d = 128 needs about 35 MiB).
 *   Races    every call on one GPU shares that GPU's scratch: calls whose
 *            work overlaps on one GPU (different streams, or host threads
 *            enqueueing on different streams) race and give undefined
 *            results.  Calls on one stream run in order and are safe.
 *   State    the scratch keeps the last call's contents; each call clears
 *            what it needs cleared itself (with kernels, not memsets).
 *   Errors   as fk_update_bias, plus FK_EHIP if the scratch's address
 *            cannot be found on the device.  fk_error_count does not apply
 *            (there is no workspace to pass).
 */
fk_status fk_update_bias_noalloc(const fk_problem* p, const void* X, const int32_t* labels,
                                 const float* C_prev, float* C_next, void* C_next_lowp,
                                 int32_t* counts, float* bias_next, void* stream);

/*
 * fk_lloyd -- max_iters Lloyd iterations (papernotes.org notes, 整体框架
 * flowchart: assign, update, repeat until converged or the iteration limit).
 * C [B][K][d] fp32: initial centroids on entry, final ones on exit.  Each
 * assignment reads C rounded to nearest even in the problem dtype.  labels
 * [B][N] and counts [B][K] are those of the last assignment.  tol > 0 stops
 * after the first iteration whose largest squared centroid move
 * max_{b,k} |c_new - c_old|^2 is <= tol; tol == 0 runs exactly max_iters.
 * n_iter (host, may be NULL) receives the number of iterations run.  With
 * tol == 0 and n_iter == NULL nothing synchronises; otherwise the call
 * synchronises the stream once per iteration.
 */
fk_status fk_lloyd(const fk_problem* p, const void* X, float* C, int32_t* labels,
                   int32_t* counts, int max_iters, float tol, int* n_iter, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * fk_lloyd_streamed -- fk_lloyd for inputs held in host memory
 * (papernotes.org notes, 关键设计 3: chunks of the point set move from host
 * to device on asynchronous streams, ping-pong, overlapped with the assign
 * and update work, so device memory no longer bounds N).
 *   X_host [B][N][d] problem dtype, PINNED host memory (hipHostMalloc);
 *   chunk_points points per chunk (the last chunk of a problem may be
 *     shorter); the workspace holds two chunk buffers, see
 *     fk_workspace_size(p, chunk_points, ...);
 *   C, labels, counts as in fk_lloyd (device memory); max_iters iterations
 *     are run (no tolerance stop);
 *   compute_stream runs the kernels, copy_stream the host-to-device copies
 *     (they may be the same stream, then nothing overlaps).
 * Per iteration each chunk is copied once; chunk j+1 is copied while chunk
 * j is assigned and reduced; sums and counts accumulate over all chunks and
 * the centroids are finalized once per iteration.  Work already queued on
 * compute_stream completes before the first copy starts.  Returns FK_EHOST
 * when stream events cannot be created.
 */
fk_status fk_lloyd_streamed(const fk_problem* p, const void* X_host, int64_t chunk_points,
                            float* C, int32_t* labels, int32_t* counts, int max_iters, void* ws,
                            size_t ws_bytes, void* compute_stream, void* copy_stream);

/*
 * fk_error_count -- number of out-of-range labels (summed over the B
 * problems) skipped by the most recent fk_sort_labels / fk_update /
 * fk_lloyd that used workspace ws.  Synchronises the stream.  *count is a
 * host pointer.
 */
fk_status fk_error_count(const fk_problem* p, const void* ws, size_t ws_bytes, int64_t* count,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FK_H */
