/*
 * dlrm_synth.h -- device-side synthetic table fill (input generation only).
 *
 * Writes the counter-hash table contents that the package's seeded generator
 * module defines, so that tables too large to build on the host (tens to
 * hundreds of GB) are created directly in HBM.  Holds none of the method's
 * arithmetic.  Element (t, r, d) of a table with scale a = fp32(1/sqrt(V_t)):
 *
 *     c = (t << 50) | (r << 12) | d
 *     h = splitmix64(seed ^ splitmix64(c))       (Steele, Lea & Flood 2014)
 *     x = fp32(2*(h >> 40) - 2^24) * 2^-24 * a   (last multiply rounds once, RN)
 *
 * stored as fp32, or as bf16 by round-to-nearest-even.
 *
 *   table  device pointer [rows][D] of dtype (DLRM_F32 / DLRM_BF16), 16-byte aligned
 *   rows < 2^38, D < 4096 with D*sizeof(elem) % 16 == 0, t < 2^14
 * Enqueues on `stream`; returns DLRM_OK or a DLRM_ERR_* code (dlrm_sparse.h).
 */
#ifndef DLRM_SYNTH_H
#define DLRM_SYNTH_H

#include "dlrm_sparse.h"

#ifdef __cplusplus
extern "C" {
#endif

int dlrm_synth_fill_table(void *table, int32_t dtype, int64_t rows, int32_t D, int32_t t,
                          uint64_t seed, float scale, dlrm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DLRM_SYNTH_H */
