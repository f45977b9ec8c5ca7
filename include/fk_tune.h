/*
 * fk_tune.h -- launch one chosen shape of the fused assign kernel, for
 * checking the library's own choice (fk_assign picks the shape from the
 * register and LDS budgets) against an exhaustive sweep.  Exported by the
 * same library as fk.h; conventions are those of fk.h.
 *
 * The pages this library follows (papernotes.org notes "Flash-KMeans: Fast
 * and Memory-Efficient Exact K-Means", 关键设计 3) describe choosing the
 * kernel's tile sizes from a hardware model instead of a search; this entry
 * point is the search.
 */
#ifndef FK_TUNE_H
#define FK_TUNE_H

#include "fk.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fk_assign_variant -- fk_assign_with_bias with an explicit kernel shape:
 *   point_blocks  16-point column blocks per wave: 1, 2, 4 or 8;
 *   waves         waves per workgroup: 2, 4 or 8;
 *   grid_wgs      workgroups launched (each then takes several blocks of
 *                 points in turn); 0 = one workgroup per block of points.
 * Labels are identical to fk_assign_with_bias for every shape.  fp16
 * problems with d = 64, 128 or 256 and K >= 32 only (FK_EUNSUPPORTED
 * otherwise).  Shapes beyond the register budget run, slowly (spills).
 */
fk_status fk_assign_variant(const fk_problem* p, const void* X, const void* C, const float* bias,
                            int32_t* labels, int point_blocks, int waves, int64_t grid_wgs,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FK_TUNE_H */
