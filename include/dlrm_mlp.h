/*
 * dlrm_mlp.h -- C ABI of the dense layers either side of the sparse path (MI355X, gfx950).
 *
 * What the calls compute (robocikowo.com "DLRM", paragraph "Forward pass": stage (1) the bottom
 * MLP, fully connected layers with ReLU producing the D-wide dense vector; stage (4) the top MLP
 * on [interaction values | dense vector], fully connected layers with a sigmoid at the end; the
 * training sentence: cross-entropy against the clicks, SGD/Adagrad; and its paragraph on the top
 * MLP).  The pages give no layer widths and no precision; the reading taken here: weights and
 * activations stored in bf16, products accumulated in fp32, fp32 master weights updated by SGD.
 *
 * Conventions: as dlrm_sparse.h (device pointers unless marked, caller-owned buffers, calls
 * enqueue on `stream` and return, arguments validated before anything is enqueued).  All
 * matrices are row-major with rows packed (leading dimension = the column count).
 *
 * The GEMMs of the linear layers run in hipBLASLt (bf16 inputs, fp32 accumulation).  The library
 * keeps one hipBLASLt handle per device and a cache of the algorithm chosen for each GEMM shape
 * (created on first use, mutex-guarded, kept until the process ends); the GEMM scratch is the
 * caller's workspace.  The first call for a GEMM shape times up to 8 candidate algorithms on the
 * caller's stream and waits for them (not graph-capturable); later calls only enqueue.
 */
#ifndef DLRM_MLP_H
#define DLRM_MLP_H

#include <stddef.h>
#include <stdint.h>

#include "dlrm_sparse.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Activation of a linear layer. */
typedef enum { DLRM_ACT_NONE = 0, DLRM_ACT_RELU = 1 } dlrm_activation;

/* Bytes of workspace the linear-layer calls need for an M x N layer output with K inputs (GEMM
 * scratch, the per-block partial sums of the bias gradient, and the per-slice partial weight
 * gradients: the weight-gradient GEMM sums over the M rows in up to 8 slices of >= 2048 rows, run
 * as one batched GEMM, then adds the slices in order).  0 on invalid sizes. */
size_t dlrm_linear_workspace_size(int64_t M, int32_t N, int32_t K);

/*
 * Fully connected layer, forward:  y = act(x W^T + b)  ([P5] stages (1) and (4)).
 *   x [M][K] bf16;  W [N][K] bf16 (one output unit per row);  b [N] fp32
 *   y [M][N] of y_dtype: DLRM_BF16 (rounded to nearest even) or DLRM_F32
 *   Limits: M >= 1, 1 <= N, K <= 65536, N and K multiples of 8 (16-byte rows); buffers 16-byte
 *   aligned; workspace >= dlrm_linear_workspace_size(M, N, K) bytes, 256-byte aligned.
 */
int dlrm_linear_fwd(const uint16_t *x, const uint16_t *W, const float *b, int64_t M, int32_t N,
                    int32_t K, int32_t act, void *y, int32_t y_dtype, void *workspace,
                    size_t workspace_bytes, dlrm_stream_t stream);

/*
 * Fully connected layer, backward (the derivative of dlrm_linear_fwd; the pages give only the
 * forward map and say it is trained by gradient descent).  With dy the gradient of y:
 *   dz = dy * [y > 0] for DLRM_ACT_RELU (y > 0 exactly where the pre-activation is), else dy
 *   dx = dz W  [M][K] fp32 (skipped when dx is NULL: the first layer)
 *   dW = dz^T x  [N][K] fp32;   db = sum over rows of dz  [N] fp32 (fp32 dz, fixed order)
 * The two GEMMs take dz rounded to bf16, written to dz_bf16 [M][N] (caller-owned scratch).
 *   dy [M][N] fp32;  y [M][N] of y_dtype (the forward output);  x, W as in the forward.
 */
int dlrm_linear_bwd(const float *dy, const void *y, int32_t y_dtype, int32_t act, const uint16_t *x,
                    const uint16_t *W, int64_t M, int32_t N, int32_t K, uint16_t *dz_bf16, float *dx,
                    float *dW, float *db, void *workspace, size_t workspace_bytes,
                    dlrm_stream_t stream);

/* Bytes of workspace dlrm_bce_head needs (per-block partial sums).  0 on invalid sizes. */
size_t dlrm_bce_head_workspace_size(int64_t M, int32_t K);

/*
 * The last layer of the top MLP, one unit with a sigmoid, and the mean binary cross-entropy
 * against the clicks ([P5] stage (4) and the training sentence), forward and backward at once:
 *   z = x w + b,  p = 1 / (1 + e^-z)
 *   loss = (1/M) sum_m [ max(z,0) - z t + log(1 + e^-|z|) ]   (= -(t log p + (1-t) log(1-p)))
 *   dz = (p - t) / M;  dx = dz w^T [M][K] fp32;  dw = x^T dz [K] fp32;  db = sum dz [1] fp32
 *   x [M][K] bf16;  w [K] bf16;  b [1] fp32;  t [M] fp32 (0 or 1)
 *   p [M], loss [1], dx, dw, db: fp32 outputs (written in full; sums in a fixed order)
 *   Limits: K % 8 == 0, K <= 4096; workspace >= dlrm_bce_head_workspace_size(M, K), 256-aligned.
 */
int dlrm_bce_head(const uint16_t *x, const uint16_t *w, const float *b, const float *t, int64_t M,
                  int32_t K, float *p, float *loss, float *dx, float *dw, float *db,
                  void *workspace, size_t workspace_bytes, dlrm_stream_t stream);

/*
 * SGD on a dense parameter ([P5] training sentence):  w32[i] -= lr * g[i];  when w16 is not NULL
 * its bf16 copy is refreshed, w16[i] = bf16(w32[i]) rounded to nearest even.  n >= 0.
 */
int dlrm_sgd_dense(float *w32, uint16_t *w16, const float *g, int64_t n, float lr,
                   dlrm_stream_t stream);

/*
 * The SGD of dlrm_sgd_dense on `count` parameters at once (one launch, the same arithmetic and
 * bits): for each i, w32[i][e] -= lr * g[i][e] for e < n[i], and the bf16 copy w16[i] refreshed
 * when w16 is not NULL and w16[i] is not NULL.  w32, w16, g, n are host arrays of count device
 * pointers / sizes; 0 <= count <= 64; n[i] >= 0.  The parameters must not overlap.
 */
int dlrm_sgd_dense_multi(int32_t count, float *const *w32, uint16_t *const *w16, const float *const *g,
                         const int64_t *n, float lr, dlrm_stream_t stream);

/*
 * Row copy with a type change and zero padding, to give a matrix the 16-byte rows the GEMMs need
 * (13 dense features -> 16, the 479-wide interaction output -> 480) or to drop the padding again:
 *   dst[m][c] = src[m][c] for c < cols,  0 for cols <= c < dst_cols
 *   src [M][src_ld] of src_dtype, dst [M][dst_cols] of dst_dtype (DLRM_F32 or DLRM_BF16; fp32 ->
 *   bf16 rounds to nearest even).  cols <= src_ld, cols <= dst_cols.
 */
int dlrm_cast_rows(const void *src, int32_t src_dtype, int64_t src_ld, int64_t M, int32_t cols,
                   void *dst, int32_t dst_dtype, int32_t dst_cols, dlrm_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DLRM_MLP_H */
