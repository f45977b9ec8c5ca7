/*
 * oracle.c -- plain, slow, fp64 CPU reference for one exact Lloyd k-means
 * iteration (assign + update), batched over B independent problems.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU library.
 *
 * What is computed, and where the pages say so:
 *
 *  - One Lloyd step is an assignment followed by a centroid update: every point
 *    goes to its nearest centroid, then every centroid becomes the mean of the
 *    points assigned to it.  (7minutos.es article on Flash-KMeans, section
 *    "¿Qué es Flash-KMeans?", the two stages of a standard Lloyd iteration;
 *    its interactive explainer: one step = one assignment + one update;
 *    tilnote.io Flash-KMeans overview, opening paragraph.)
 *  - The method is exact: its output equals standard Lloyd, so the reference
 *    is the textbook definition, not the tiled algorithm.  (7minutos.es
 *    article, "¿Qué es Flash-KMeans?" and "Conclusiones clave"; papernotes.org
 *    "Flash-KMeans: Fast and Memory-Efficient Exact K-Means", 一句话总结 and
 *    亮点与洞察.)
 *  - Inputs X (N x d), C (K x d), output label vector a.  (papernotes.org
 *    notes, 方法详解 / 整体框架.)
 *  - Assignment keeps a running minimum m <- +inf and index a <- -1 and merges
 *    with min/argmin.  (papernotes.org notes, 关键设计 1, FlashAssign merge
 *    equation.)  The pages fix no tie rule; the reading taken here is: the
 *    lowest index among exactly equal distances wins (centroids are scanned
 *    in ascending order and replaced only on a strictly smaller distance).
 *  - Update sums the member vectors and counts per cluster, then divides.
 *    (papernotes.org notes, 关键设计 2, the per-cluster (s_k, n_k) merge.)
 *    The pages say nothing about empty clusters; the reading taken here is:
 *    an empty cluster keeps its previous centroid unchanged.
 *  - Iterate until converged or a maximum number of steps.  (papernotes.org
 *    notes, 整体框架 flowchart.)  Here: a fixed number of steps.
 *
 * Distances are the plain definition sum_j (x_j - c_j)^2 in fp64, summed over
 * j in ascending order; no expansion, blocking or reordering.  Stored 16-bit
 * and 32-bit floats are decoded to fp64 exactly by this file's own decoders.
 *
 * Dtype codes: 0 = fp32, 1 = fp16 (IEEE binary16), 2 = bf16, 3 = fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI 1

int oracle_abi_version(void) { return ORACLE_ABI; }

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * Exact decoding of stored floats to fp64.
 * binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
 * ------------------------------------------------------------------------- */
static double decode_small_float(uint32_t bits, int ebits, int fbits) {
    const uint32_t emask = (1u << ebits) - 1u;
    const int bias = (int)(emask >> 1);
    const uint32_t sign = (bits >> (ebits + fbits)) & 1u;
    const uint32_t e = (bits >> fbits) & emask;
    const uint32_t f = bits & ((1u << fbits) - 1u);
    double mag;
    if (e == 0) {
        /* zero or subnormal: f * 2^(1 - bias - fbits) */
        mag = ldexp((double)f, 1 - bias - fbits);
    } else if (e == emask) {
        mag = (f == 0) ? INFINITY : NAN;
    } else {
        /* normal: (2^fbits + f) * 2^(e - bias - fbits) */
        mag = ldexp((double)((1u << fbits) + f), (int)e - bias - fbits);
    }
    return sign ? -mag : mag;
}

static double decode_one(int dtype, const void* base, int64_t idx) {
    switch (dtype) {
        case 0: return (double)((const float*)base)[idx];
        case 1: return decode_small_float(((const uint16_t*)base)[idx], 5, 10);
        case 2: return decode_small_float(((const uint16_t*)base)[idx], 8, 7);
        default: return ((const double*)base)[idx];
    }
}

void oracle_decode(int dtype, const void* src, int64_t n, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = decode_one(dtype, src, i);
}

/* ---------------------------------------------------------------------------
 * Round-to-nearest-even encoding of an fp32 value into a narrower binary
 * format with p significand bits (implicit bit included).
 *
 * Write v = m * 2^e with 0.5 <= |m| < 1 (frexp).  Representable neighbours of
 * v are multiples of the quantum 2^(max(e, e_min) - p), where e_min is frexp's
 * exponent of the smallest normal number; below it the spacing is fixed
 * (subnormals).  v / quantum is exact in fp64 and rint() rounds it to the
 * nearest integer with ties to even (the default rounding mode).  A result
 * above the largest finite value becomes infinity.
 * ------------------------------------------------------------------------- */
static uint16_t encode_rne(float xf, int ebits, int fbits) {
    const int p = fbits + 1;
    const int bias = (1 << (ebits - 1)) - 1;
    const int e_min = 2 - bias;          /* frexp exponent of 2^(1-bias) */
    const uint16_t sign = signbit(xf) ? (uint16_t)(1u << (ebits + fbits)) : 0;
    const uint16_t inf_bits = (uint16_t)(((1u << ebits) - 1u) << fbits);
    double v = fabs((double)xf);
    if (isnan(xf)) return (uint16_t)(sign | inf_bits | (1u << (fbits - 1)));
    if (isinf(xf)) return (uint16_t)(sign | inf_bits);
    if (v == 0.0) return sign;
    int e;
    (void)frexp(v, &e);
    const int qexp = (e > e_min ? e : e_min) - p;
    double r = ldexp(rint(ldexp(v, -qexp)), qexp);
    /* largest finite: (2 - 2^(1-p)) * 2^bias */
    const double maxfin = ldexp(2.0 - ldexp(1.0, 1 - p), bias);
    if (r > maxfin) return (uint16_t)(sign | inf_bits);
    if (r == 0.0) return sign;
    (void)frexp(r, &e);
    uint32_t bits;
    if (e >= e_min) {
        /* normal: r = (2^fbits + f) * 2^(e - 1 - fbits), exponent field e - 1 + bias */
        uint32_t f = (uint32_t)(ldexp(r, fbits + 1 - e) - ldexp(1.0, fbits));
        bits = ((uint32_t)(e - 1 + bias) << fbits) | f;
    } else {
        /* subnormal: r = f * 2^(1 - bias - fbits) */
        bits = (uint32_t)ldexp(r, bias - 1 + fbits);
    }
    return (uint16_t)(sign | bits);
}

void oracle_encode_f16_rne(const float* src, int64_t n, uint16_t* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = encode_rne(src[i], 5, 10);
}

void oracle_encode_bf16_rne(const float* src, int64_t n, uint16_t* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = encode_rne(src[i], 8, 7);
}

/* ---------------------------------------------------------------------------
 * Assignment.
 *
 * For each requested point (b, i): scan k = 0..K-1 in ascending order,
 * dist = sum_j (x_ij - c_kj)^2 in fp64 (j ascending), keep the smallest (d1)
 * and its index (replace only when strictly smaller), and the second smallest
 * over the remaining centroids (d2).  An exact tie leaves d2 == d1.
 *
 * rows == NULL: all B*N points, outputs indexed b*N + i.
 * rows != NULL: only the flattened point ids rows[0..nrows), outputs indexed
 * 0..nrows-1.  (Used to check sampled outputs of large problems one by one.)
 * ------------------------------------------------------------------------- */
void oracle_assign(int dtype_x, int dtype_c, int64_t B, int64_t N, int64_t K, int64_t d,
                   const void* X, const void* C, const int64_t* rows, int64_t nrows,
                   int32_t* labels, double* d1_out, double* d2_out, int nthreads) {
    const int64_t npts = rows ? nrows : B * N;
    double* Cd = (double*)malloc(sizeof(double) * (size_t)(B * K * d));
    oracle_decode(dtype_c, C, B * K * d, Cd);
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double* x = (double*)malloc(sizeof(double) * (size_t)d);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
        for (int64_t t = 0; t < npts; ++t) {
            const int64_t p = rows ? rows[t] : t;   /* flattened point id b*N + i */
            const int64_t b = p / N;
            for (int64_t j = 0; j < d; ++j) x[j] = decode_one(dtype_x, X, p * d + j);
            double best = INFINITY, second = INFINITY;
            int32_t arg = -1;
            for (int64_t k = 0; k < K; ++k) {
                const double* c = Cd + (b * K + k) * d;
                double dist = 0.0;
                for (int64_t j = 0; j < d; ++j) {
                    const double diff = x[j] - c[j];
                    dist += diff * diff;
                }
                if (dist < best) {
                    second = best;
                    best = dist;
                    arg = (int32_t)k;
                } else if (dist < second) {
                    second = dist;
                }
            }
            labels[t] = arg;
            if (d1_out) d1_out[t] = best;
            if (d2_out) d2_out[t] = second;
        }
        free(x);
    }
    free(Cd);
}

/* ---------------------------------------------------------------------------
 * Squared distance of given (point, centroid) pairs, the same plain
 * definition as in oracle_assign: sum_j (x_pj - c_kj)^2, fp64, j ascending.
 * points[t] is a flattened point id b*N + i, cents[t] a centroid index of the
 * same problem.  Used to check that a label chosen among near-ties is still
 * near-optimal.
 * ------------------------------------------------------------------------- */
void oracle_pair_dist(int dtype_x, int dtype_c, int64_t B, int64_t N, int64_t K, int64_t d,
                      const void* X, const void* C, const int64_t* points, const int32_t* cents,
                      int64_t npairs, double* out) {
    (void)B;
    for (int64_t t = 0; t < npairs; ++t) {
        const int64_t p = points[t];
        const int64_t b = p / N;
        const int64_t k = cents[t];
        double dist = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            const double diff = decode_one(dtype_x, X, p * d + j) -
                                decode_one(dtype_c, C, (b * K + k) * d + j);
            dist += diff * diff;
        }
        out[t] = dist;
    }
}

/* ---------------------------------------------------------------------------
 * Update from a given label vector.
 *
 * counts[b,k] = number of i with labels[b,i] == k (exact integers).
 * sums accumulate member vectors in fp64 in ascending i.
 * C_next[b,k] = sums / counts when counts > 0, else C_prev[b,k] unchanged.
 * Returns the number of labels outside [0, K) (those points are skipped).
 * ------------------------------------------------------------------------- */
int64_t oracle_update(int dtype_x, int dtype_c, int64_t B, int64_t N, int64_t K, int64_t d,
                      const void* X, const int32_t* labels, const void* C_prev,
                      int64_t* counts, double* C_next, int nthreads) {
    int64_t bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for reduction(+ : bad) schedule(static, 1)
#endif
    for (int64_t b = 0; b < B; ++b) {
        double* sums = (double*)calloc((size_t)(K * d), sizeof(double));
        int64_t* cnt = counts + b * K;
        for (int64_t k = 0; k < K; ++k) cnt[k] = 0;
        for (int64_t i = 0; i < N; ++i) {
            const int32_t a = labels[b * N + i];
            if (a < 0 || a >= K) { ++bad; continue; }
            cnt[a] += 1;
            for (int64_t j = 0; j < d; ++j)
                sums[a * d + j] += decode_one(dtype_x, X, (b * N + i) * d + j);
        }
        for (int64_t k = 0; k < K; ++k) {
            for (int64_t j = 0; j < d; ++j) {
                const int64_t o = (b * K + k) * d + j;
                C_next[o] = cnt[k] > 0 ? sums[k * d + j] / (double)cnt[k]
                                       : decode_one(dtype_c, C_prev, o);
            }
        }
        free(sums);
    }
    return bad;
}

/* ---------------------------------------------------------------------------
 * Free-running Lloyd in fp64: T iterations of assign then update, centroids
 * kept in fp64 throughout.  C is the fp64 initial centroids on entry and
 * C^(T) on exit; labels/counts are those of the last assignment;
 * objective[t] = sum of nearest squared distances at assignment t.
 * ------------------------------------------------------------------------- */
void oracle_lloyd(int dtype_x, int64_t B, int64_t N, int64_t K, int64_t d, const void* X,
                  double* C, int64_t T, int32_t* labels, int64_t* counts, double* objective,
                  int nthreads) {
    double* d1 = (double*)malloc(sizeof(double) * (size_t)(B * N));
    double* Cn = (double*)malloc(sizeof(double) * (size_t)(B * K * d));
    for (int64_t t = 0; t < T; ++t) {
        oracle_assign(dtype_x, 3, B, N, K, d, X, C, NULL, 0, labels, d1, NULL, nthreads);
        double J = 0.0;
        for (int64_t p = 0; p < B * N; ++p) J += d1[p];
        if (objective) objective[t] = J;
        oracle_update(dtype_x, 3, B, N, K, d, X, labels, C, counts, Cn, nthreads);
        memcpy(C, Cn, sizeof(double) * (size_t)(B * K * d));
    }
    free(Cn);
    free(d1);
}
