/*
 * dlrm_sparse.h -- C ABI of the DLRM sparse hot path for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute is defined on these pages:
 *   [P5] robocikowo.com "DLRM" (technologie-ai): paragraph "Forward pass",
 *        stages (2) lookup, (3) pairwise dots / upper triangle, (4) the
 *        concatenation with the bottom-MLP output; the paragraph on the
 *        embedding tables (E_i: V_i x D, indexed lookup); the paragraph on
 *        the interaction layer (N vectors = bottom-MLP output + N-1
 *        embeddings, N(N-1)/2 values); the training sentence (SGD/Adagrad).
 *   [P2] notes.helloworld.co.in "Deep Learning Recommendation Model (DLRM)",
 *        section "The architecture".
 *   [P4] vinsonli.com "The embedding table is the model".
 *   [P1] technolynx.com "DLRM explained", section "How does DLRM actually work?".
 * Where the pages leave a step open (bag pooling, triu order, backward,
 * row-wise Adagrad), the reading taken is stated at the call.
 *
 * Conventions common to every call
 *   - Pointers are DEVICE pointers unless marked (host).  Host arrays are
 *     read before the call returns.
 *   - The caller allocates and owns every device buffer, including the
 *     workspace, and keeps it alive until the work on `stream` completes.
 *     The library allocates no device memory and keeps no mutable state
 *     (apart from the opt-in kernel timing record, dlrm_trace_*), so calls on
 *     different streams may run concurrently on distinct buffers.
 *   - Every call enqueues on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns without waiting, except with DLRM_FLAG_CHECK_INDICES, which
 *     synchronises the stream to report the result of the check.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing has been enqueued and outputs are untouched.  A failed
 *     launch returns DLRM_ERR_HIP.
 *   - Bags are table-major: bag (t, b) has id t*B + b; offsets has T*B + 1
 *     entries, offsets[0] = 0, offsets[T*B] = nnz, non-decreasing, and every
 *     index of a bag of table t lies in [0, rows[t]).  Breaking these is
 *     undefined behaviour unless DLRM_FLAG_CHECK_INDICES is given.
 *   - Outputs must not alias inputs.
 *   - Limits: 1 <= T <= 64; 1 <= D <= 512 with D*sizeof(elem) a multiple of
 *     16 bytes (D % 4 == 0 for fp32 tables, D % 8 == 0 for bf16); T*B < 2^31;
 *     nnz < 2^31; table pointers 16-byte aligned; indices/offsets 8-byte
 *     aligned; float buffers 16-byte aligned.
 */
#ifndef DLRM_SPARSE_H
#define DLRM_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t *dlrm_stream_t;

/* Table element type (and pooled output type of emb_bag_fwd_ex).  bf16 values are the upper
 * 16 bits of an fp32. */
typedef enum { DLRM_F32 = 0, DLRM_BF16 = 1 } dlrm_dtype;

/* Integer type of indices and offsets (the *_ex / *_update calls). */
typedef enum { DLRM_INDEX_I64 = 0, DLRM_INDEX_I32 = 1 } dlrm_index_type;

/* Update rule of emb_bag_bwd_update. */
typedef enum { DLRM_OPT_ADAGRAD = 0, DLRM_OPT_SGD = 1 } dlrm_optimizer;

enum {
    DLRM_OK = 0,
    DLRM_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment          */
    DLRM_ERR_UNSUPPORTED = -2, /* valid but outside the library's limits         */
    DLRM_ERR_HIP = -3,         /* a HIP launch or runtime call failed            */
    DLRM_ERR_INDEX_RANGE = -4, /* CHECK_INDICES found a bad index or offset      */
    DLRM_ERR_WORKSPACE = -5    /* workspace missing or smaller than required     */
};

/* Validate offsets and indices on the device before the work (a debug aid):
 * the call synchronises `stream` and returns DLRM_ERR_INDEX_RANGE if any
 * offset decreases, offsets[0] != 0, offsets[T*B] != nnz, or an index lies
 * outside its table.  With this flag the call is not graph-capturable. */
#define DLRM_FLAG_CHECK_INDICES 1u

/*
 * Embedding-bag lookup with sum pooling ([P5] stage (2) and the table
 * paragraph; [P1] one lookup per sparse feature; [P2] the vectors come out
 * at equal width D).  A multi-valued feature is a bag of indices; its rows
 * are summed, or weighted by one fp32 weight per lookup:
 *
 *     out[b][t][d] = sum_{j in [offsets[t*B+b], offsets[t*B+b+1])} w_j * E_t[indices[j]][d]
 *
 * w_j = 1 when per_sample_weights is NULL; an empty bag gives zeros.
 * Accumulation is fp32 (bf16 rows widen exactly).  The summation order is
 * fixed, so results are bitwise reproducible.
 *
 *   tables  (host) [T] device pointers, table t row-major [rows[t]][D] of `dtype`
 *   rows    (host) [T] row counts V_t >= 1
 *   indices [nnz] int64; offsets [T*B+1] int64; per_sample_weights [nnz] fp32 or NULL
 *   out     [B][T][D] fp32 (written in full)
 */
int emb_bag_fwd(const void *const *tables, const int64_t *rows, int32_t T, int32_t D,
                int32_t dtype, const int64_t *indices, const int64_t *offsets,
                const float *per_sample_weights, int64_t B, int64_t nnz, float *out,
                uint32_t flags, dlrm_stream_t stream);

/*
 * emb_bag_fwd with a choice of index type and pooled output type.
 *   indices, offsets: int64 (DLRM_INDEX_I64) or int32 (DLRM_INDEX_I32), same type for both,
 *                     aligned to their size
 *   out: [B][T][D] of out_dtype: DLRM_F32, or DLRM_BF16 = the fp32 pooled value rounded to
 *        nearest even (halves the output bytes); 16-byte aligned
 * Everything else as emb_bag_fwd, which is emb_bag_fwd_ex(..., DLRM_INDEX_I64, ..., DLRM_F32).
 * The pooled sums are the same fp32 values for both index types.
 */
int emb_bag_fwd_ex(const void *const *tables, const int64_t *rows, int32_t T, int32_t D,
                   int32_t dtype, const void *indices, const void *offsets, int32_t index_type,
                   const float *per_sample_weights, int64_t B, int64_t nnz, void *out,
                   int32_t out_dtype, uint32_t flags, dlrm_stream_t stream);

/*
 * Dot-product interaction, forward ([P5] stage (3) and the interaction
 * paragraph; [P2] "The architecture"; [P4]).  Per sample the N vectors are
 * the rows of X (N x D): row 0 the dense (bottom-MLP) vector, rows 1..N-1 the
 * pooled embeddings of tables 0..N-2.  The output row holds the strict upper
 * triangle of X X^T, N(N-1)/2 values listed row by row (i < j, i then j
 * ascending), followed by the dense vector ([P5] stage (4): interaction
 * values first, then the bottom-MLP output):
 *
 *     out[b] = [ <x0,x1>, <x0,x2>, ..., <x_{N-2},x_{N-1}>, dense[b][0..D-1] ]
 *
 *   dense  [B][D] fp32; pooled [B][N-1][D] fp32 (the layout emb_bag_fwd writes)
 *   out    [B][N(N-1)/2 + D] fp32
 *   Limits: 1 <= N <= 65, D % 4 == 0, D <= 512.  fp32 arithmetic.
 */
int dlrm_interact_fwd(const float *dense, const float *pooled, int64_t B, int32_t N, int32_t D,
                      float *out, dlrm_stream_t stream);

/* Gram path of dlrm_interact_fwd_ex. */
enum { DLRM_GRAM_AUTO = 0, DLRM_GRAM_MFMA = 1, DLRM_GRAM_VALU = 2 };

/*
 * dlrm_interact_fwd with the kernel chosen by the caller, for measuring one Gram path against the
 * other on the same shapes.  Same output, same arguments, plus:
 *   path  DLRM_GRAM_AUTO: dlrm_interact_fwd's own choice (the k-split VALU Gram for N <= 11 and
 *           D in {64, 128, 256}, else the fp32 matrix-core Gram);
 *         DLRM_GRAM_MFMA: the matrix-core Gram (v_mfma_f32_16x16x4_f32) for every N
 *           (DLRM_ERR_UNSUPPORTED where D is not a multiple of 16 or above 512);
 *         DLRM_GRAM_VALU: the plain-VALU Gram with X staged in LDS and 2x2 register tiles of dots
 *           (D a multiple of 16 and N*(D+4)*4 <= 64 KiB, else DLRM_ERR_UNSUPPORTED).
 * Each path sums every dot in fp32; the paths add the D products in different orders, so their
 * results agree to rounding, not bit for bit.
 */
int dlrm_interact_fwd_ex(const float *dense, const float *pooled, int64_t B, int32_t N, int32_t D,
                         float *out, int32_t path, dlrm_stream_t stream);

/*
 * Dot-product interaction, backward: the derivative of dlrm_interact_fwd
 * (the pages give the forward map and say it is trained by gradient descent,
 * [P5] training sentence).  With g = grad_out[b], G the symmetric N x N
 * matrix with zero diagonal and G[i][j] = G[j][i] = g[p(i,j)] (p the triu
 * position above):
 *
 *     dX = G X;   grad_dense[b] = dX[0] + g[P .. P+D-1];   grad_pooled[b][t] = dX[t+1]
 *
 *   grad_out [B][P+D]; dense [B][D]; pooled [B][N-1][D]  (all fp32)
 *   grad_dense [B][D]; grad_pooled [B][N-1][D]           (fp32, written in full)
 *   Same limits as the forward.
 */
int dlrm_interact_bwd(const float *grad_out, const float *dense, const float *pooled, int64_t B,
                      int32_t N, int32_t D, float *grad_dense, float *grad_pooled,
                      dlrm_stream_t stream);

/*
 * Lookup fused with the interaction, for inference ([P5] "Forward pass" stages (2)-(4) in
 * sequence: the pooled vectors of a sample go straight into the pairwise dots and the
 * concatenation).  Computes exactly dlrm_interact_fwd(dense, emb_bag_fwd(...)) -- the same
 * pooling and the same matrix-core arithmetic, so the bits are identical -- without writing
 * the pooled [B][T][D] array: each sample's N = T + 1 vectors are kept on chip.
 *
 *   tables, rows, T, D, dtype, indices, offsets, per_sample_weights, B, nnz: as emb_bag_fwd
 *   dense [B][D] fp32, 16-byte aligned
 *   out   [B][N(N-1)/2 + D] fp32: the strict upper triangle of X X^T row by row, then dense
 *   flags: DLRM_FLAG_CHECK_INDICES as for emb_bag_fwd (the check borrows 4 bytes of out)
 *   Limits: D % 16 == 0 and D*sizeof(elem) in {64, 128, 256, 512, 1024} bytes (fp32 D in
 *   {16..256}, bf16 D in {32..512}); one sample's X, N*(D+4)*4 bytes, plus the bags' offsets
 *   must fit in 64 KiB (DLRM_ERR_UNSUPPORTED otherwise; use the two calls).
 */
int emb_bag_interact_fwd(const void *const *tables, const int64_t *rows, int32_t T, int32_t D,
                         int32_t dtype, const int64_t *indices, const int64_t *offsets,
                         const float *per_sample_weights, int64_t B, int64_t nnz,
                         const float *dense, float *out, uint32_t flags, dlrm_stream_t stream);

/* Bytes of device workspace emb_bag_bwd_adagrad needs for these sizes
 * (0 on invalid sizes).  rows is a host array of T row counts.  D is an argument because part
 * of the workspace scales with it: the segment sums that cross chunk boundaries are kept as fp32
 * rows of D values, one or two per chunk, and the chunk length follows from D (a lane group of
 * D/4 lanes walks each chunk). */
size_t emb_bag_bwd_workspace_size(int32_t T, const int64_t *rows, int32_t D, int64_t B,
                                  int64_t nnz);

/*
 * Embedding backward with row-wise Adagrad, applied in place ([P5] training
 * sentence names SGD/Adagrad; the rest is the reading stated here).  The
 * pooling is linear in the table, so row r of table t receives
 *
 *     G[d] = sum over lookups j of (t, r) of  w_j * grad_pooled[b(j)][t][d]
 *
 * Steps: key_j = rowbase[t] + indices[j] (rowbase = exclusive prefix sum of
 * rows); a stable sort of the keys; unique keys and their segments; the
 * per-segment sum G (fp32, fixed order: bitwise reproducible); then, for
 * each unique row only,
 *
 *     s      <- s + (1/D) * sum_d G[d]^2        (state[t][r], fp32)
 *     E[r,d] <- E[r,d] - lr * G[d] / (sqrt(s) + eps)
 *
 * (Duchi, Hazan & Singer 2011, with one accumulator per row).  Rows that no
 * lookup touches are not written.  bf16 tables are updated in fp32 and
 * stored round-to-nearest-even.
 *
 *   tables  (host) [T] device pointers [rows[t]][D] of `dtype`, updated in place
 *   state   (host) [T] device pointers [rows[t]] fp32, updated in place
 *   rows    (host) [T]; sum of rows must be <= 2^32
 *   indices, offsets, per_sample_weights: as emb_bag_fwd (weights may be NULL)
 *   grad_pooled [B][T][D] fp32
 *   workspace: >= emb_bag_bwd_workspace_size(T, rows, D, B, nnz) bytes, 256-byte aligned
 *   Optional outputs (written when non-NULL):
 *     unique_keys_out     [nnz] int64: the U distinct keys, ascending (first U entries)
 *     segment_offsets_out [nnz+1] int64: first sorted position of each key; entry U = nnz
 *     sorted_pos_out      [nnz] int32: original position of each sorted position
 *     num_unique_out      [1] int64: U
 *   Limits: D in [4, 512], a multiple of 4 up to 256 and of 8 above (bf16: a multiple of 8),
 *   so every row is a multiple of 16 bytes as in the forward, except fp32 rows of 260-508
 *   values that are an odd multiple of 4 (unsupported).  The segment sums run on lane groups
 *   of D/4 lanes (D/8 above 256) rounded up to a power of two, so that groups tile the 64-lane
 *   wavefront: the group sums are DPP/permute trees inside the group, and segment starts are
 *   read from the wave's ballot mask by group.
 *   Keys are 32-bit: the sum of rows must be at most 2^32.
 */
int emb_bag_bwd_adagrad(void *const *tables, float *const *state, const int64_t *rows, int32_t T,
                        int32_t D, int32_t dtype, const int64_t *indices, const int64_t *offsets,
                        const float *per_sample_weights, int64_t B, int64_t nnz,
                        const float *grad_pooled, float lr, float eps, void *workspace,
                        size_t workspace_bytes, int64_t *unique_keys_out,
                        int64_t *segment_offsets_out, int32_t *sorted_pos_out,
                        int64_t *num_unique_out, uint32_t flags, dlrm_stream_t stream);

/*
 * Embedding backward with a choice of update rule and index type ([P5] training sentence: SGD
 * or Adagrad).  The row gradients G are emb_bag_bwd_adagrad's (same sort, segments and fixed
 * summation order), then for each touched row:
 *   DLRM_OPT_ADAGRAD: the row-wise Adagrad step of emb_bag_bwd_adagrad (state required);
 *   DLRM_OPT_SGD:     E[r,d] <- E[r,d] - lr * G[d]   (state may be NULL; eps is ignored).
 *   indices, offsets: index_type as in emb_bag_fwd_ex.
 * Everything else as emb_bag_bwd_adagrad, which is
 * emb_bag_bwd_update(..., DLRM_INDEX_I64, ..., DLRM_OPT_ADAGRAD, ...).
 */
int emb_bag_bwd_update(void *const *tables, float *const *state, const int64_t *rows, int32_t T,
                       int32_t D, int32_t dtype, const void *indices, const void *offsets,
                       int32_t index_type, const float *per_sample_weights, int64_t B, int64_t nnz,
                       const float *grad_pooled, int32_t optimizer, float lr, float eps,
                       void *workspace, size_t workspace_bytes, int64_t *unique_keys_out,
                       int64_t *segment_offsets_out, int32_t *sorted_pos_out,
                       int64_t *num_unique_out, uint32_t flags, dlrm_stream_t stream);

/*
 * The embedding backward in two halves, so that the first can run while the gradient it does
 * not need is still being computed (emb_bag_bwd_update is emb_bag_bwd_plan followed by
 * emb_bag_bwd_apply on one stream, with the same results bit for bit).
 *
 * emb_bag_bwd_plan: everything that reads only the batch -- the keys, their stable sort (with
 * the lookup positions, grad rows and weights as payloads), the unique keys and segments --
 * left in `workspace` for emb_bag_bwd_apply.  It reads no table, state or gradient.
 *   Arguments as emb_bag_bwd_update (same limits, same optional integer outputs, same flags);
 *   the workspace is sized by emb_bag_bwd_workspace_size for the same rows, D, B, nnz.
 *
 * emb_bag_bwd_apply: the per-segment gradient sums and the update of emb_bag_bwd_update, from
 * a workspace that a completed emb_bag_bwd_plan with the same rows, D, B and nnz filled
 * (ordering the two across streams is the caller's: an event, or one stream).
 *   weighted: nonzero iff the plan was given per-sample weights
 *   segment_offsets: the plan's segment_offsets_out if it had one, else NULL (the copy in the
 *     workspace is used)
 *   tables, state, dtype, grad_pooled, optimizer, lr, eps: as emb_bag_bwd_update
 * The plan is left unchanged, so it can be applied again (to other tables or another
 * gradient of the same batch); applications of one workspace must not overlap in time.
 */
int emb_bag_bwd_plan(const int64_t *rows, int32_t T, int32_t D, const void *indices,
                     const void *offsets, int32_t index_type, const float *per_sample_weights,
                     int64_t B, int64_t nnz, void *workspace, size_t workspace_bytes,
                     int64_t *unique_keys_out, int64_t *segment_offsets_out,
                     int32_t *sorted_pos_out, int64_t *num_unique_out, uint32_t flags,
                     dlrm_stream_t stream);

int emb_bag_bwd_apply(void *const *tables, float *const *state, const int64_t *rows, int32_t T,
                      int32_t D, int32_t dtype, int64_t B, int64_t nnz, int32_t weighted,
                      const float *grad_pooled, int32_t optimizer, float lr, float eps,
                      void *workspace, size_t workspace_bytes, const int64_t *segment_offsets,
                      dlrm_stream_t stream);

/*
 * Allocation-free embedding backward, for callers that cannot allocate device memory or hand the
 * library a workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It is emb_bag_bwd_update with the workspace taken from a fixed array of device
 * memory the library holds on each GPU it runs on (emb_bag_bwd_noalloc_max_bytes() = 64 MiB,
 * kept until the process ends); the results are emb_bag_bwd_update's, bit for bit.
 *   Arguments: as emb_bag_bwd_update, without the workspace.
 *   A batch whose workspace (emb_bag_bwd_workspace_size) exceeds the array is refused with
 *   DLRM_ERR_WORKSPACE before anything is enqueued (at D = 128 about 1.17M lookups fit; the
 *   one-hot training batch of 26 tables x 2048 samples needs 3.7 MiB).
 *   Every call on one GPU uses that GPU's single array: calls that overlap in time on one GPU
 *   (two streams, two host threads) race, and the caller must order them.  The first call on a
 *   device looks the array's address up there; no call allocates memory.
 */
int emb_bag_bwd_update_noalloc(void *const *tables, float *const *state, const int64_t *rows,
                               int32_t T, int32_t D, int32_t dtype, const void *indices,
                               const void *offsets, int32_t index_type,
                               const float *per_sample_weights, int64_t B, int64_t nnz,
                               const float *grad_pooled, int32_t optimizer, float lr, float eps,
                               int64_t *unique_keys_out, int64_t *segment_offsets_out,
                               int32_t *sorted_pos_out, int64_t *num_unique_out, uint32_t flags,
                               dlrm_stream_t stream);

/* Bytes of the fixed device array emb_bag_bwd_update_noalloc works in. */
size_t emb_bag_bwd_noalloc_max_bytes(void);

/* Static description of a status code. */
const char *dlrm_status_string(int status);

/*
 * Kernel timing (diagnostics).  While enabled (dlrm_trace_enable(1)), every kernel the library
 * launches is bracketed by two HIP events recorded on its stream; disabled (the default), a
 * launch is unchanged apart from one atomic flag read.  dlrm_trace_read waits for the recorded
 * kernels to finish, then writes, per kernel name (sorted), the number of launches and their
 * summed milliseconds, and clears the record.  Process-wide state behind a mutex; calls that
 * record into a HIP graph capture must not have tracing enabled.
 *
 *   names    (host) max_entries * 64 chars, NUL-terminated names
 *   launches (host) [max_entries];  ms (host) [max_entries];  n_entries (host) entries written
 */
int dlrm_trace_enable(int on);
int dlrm_trace_read(int32_t max_entries, char *names, int64_t *launches, double *ms,
                    int32_t *n_entries);

#ifdef __cplusplus
}
#endif

#endif /* DLRM_SPARSE_H */
