/*
 * dlrm_probe.h -- HBM read probes (measurement context only; no part of the method).
 *
 * The lookup's speed is set by how fast rows can be read from HBM (the pages call the
 * embedding lookup memory-bandwidth bound: notes.helloworld.co.in "Deep Learning
 * Recommendation Model (DLRM)", section "Why it is mostly a systems problem").  These two
 * kernels measure the two ceilings that bound it on the running GPU, with nothing else in
 * the way: a plain streaming read, and a gather of whole rows at given indices with no
 * output written.  Each folds what it reads into one 32-bit word per workgroup (XOR), so
 * the loads cannot be dropped.
 *
 * dlrm_probe_read: reads bytes [0, nbytes) of buf once with 16-byte loads.
 *   buf    device pointer, 16-byte aligned; nbytes a multiple of 16, > 0
 *   sink   device pointer to sink_words uint32 (>= 1); the launch uses min(sink_words, 4096)
 *          workgroups and workgroup g writes sink[g]
 *
 * dlrm_probe_gather: reads row idx[i] (row_bytes bytes at buf + idx[i] * row_bytes) for
 *   i in [0, n).  An index outside [0, rows) is clamped into it, so every load stays inside
 *   the buffer.
 *   buf        device pointer to rows * row_bytes bytes, 16-byte aligned
 *   row_bytes  a multiple of 16 in [16, 1024]
 *   idx        device pointer to n int64 indices;  0 <= n < 2^31
 *   sink       as above
 *
 * Both enqueue on `stream` and return DLRM_OK, DLRM_ERR_INVALID_ARG for a bad argument
 * (checked before anything is enqueued) or DLRM_ERR_HIP for a failed launch.  The caller
 * owns every buffer.
 */
#ifndef DLRM_PROBE_H
#define DLRM_PROBE_H

#include "dlrm_sparse.h"

#ifdef __cplusplus
extern "C" {
#endif

int dlrm_probe_read(const void *buf, uint64_t nbytes, uint32_t *sink, uint32_t sink_words,
                    dlrm_stream_t stream);

int dlrm_probe_gather(const void *buf, int64_t rows, int32_t row_bytes, const int64_t *idx,
                      int64_t n, uint32_t *sink, uint32_t sink_words, dlrm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DLRM_PROBE_H */
