/*
 * CPU oracle for the DLRM sparse path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark call this code.  The GPU library never links,
 * loads or calls it, and it shares no source with the GPU library.
 *
 * Plain, slow and obviously correct: every function is the definition written
 * out as loops, accumulating in fp64 from the fp32 / bf16 inputs.  Sources:
 *
 *   [P5] robocikowo.com "DLRM" (technologie-ai), paragraph "Forward pass",
 *        stages (2) and (3) and the training sentence; the paragraphs on the
 *        embedding tables (E_i: V_i x D) and on the interaction layer.
 *   [P2] notes.helloworld.co.in "Deep Learning Recommendation Model (DLRM)",
 *        section "The architecture".
 *   [P4] vinsonli.com "The embedding table is the model" (pairwise dots
 *        between equal-width vectors, then concatenation with the dense vector).
 *   [P1] technolynx.com "DLRM explained", section "How does DLRM actually work?".
 *
 * Readings of points the pages leave open (bag reduction, triu order, the
 * concatenation order, the row-wise Adagrad form) are stated at each function.
 * Every function checks its preconditions and returns a negative code if they
 * fail; 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_OFFSETS (-2)
#define ORACLE_ERR_INDEX (-3)
#define ORACLE_ERR_NOMEM (-4)

/* Value of element (row, d) of a table stored as fp32, or as bf16 bit patterns
 * (the upper 16 bits of an fp32; widening is exact). */
static double table_value(const void *table, int dtype, int64_t row, int D, int d) {
    if (dtype == ORACLE_F32) return (double)((const float *)table)[row * (int64_t)D + d];
    uint32_t bits = (uint32_t)((const uint16_t *)table)[row * (int64_t)D + d] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* CSR preconditions: offsets start at 0, never decrease, end at nnz; every
 * index of a bag of table t lies in [0, rows[t]). */
static int check_csr(int T, const int64_t *rows, const int64_t *indices, const int64_t *offsets,
                     int64_t B) {
    int64_t nbags = (int64_t)T * B;
    if (offsets[0] != 0) return ORACLE_ERR_OFFSETS;
    for (int64_t g = 0; g < nbags; ++g) {
        if (offsets[g + 1] < offsets[g]) return ORACLE_ERR_OFFSETS;
        int64_t t = g / B;
        for (int64_t j = offsets[g]; j < offsets[g + 1]; ++j)
            if (indices[j] < 0 || indices[j] >= rows[t]) return ORACLE_ERR_INDEX;
    }
    return ORACLE_OK;
}

static int threads_or_default(int n) {
#ifdef _OPENMP
    return n > 0 ? n : omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/*
 * Embedding-bag lookup with sum pooling ([P5] stage 2 and the table paragraph:
 * each sparse feature indexes its own table E_t of shape V_t x D and yields a
 * D-wide vector; [P1] one lookup per feature).
 *
 * Reading: a multi-valued feature is a bag of indices (CSR offsets, bags in
 * table-major order: bag (t, b) has id t*B + b); the bag reduces to the plain
 * sum of its rows, or the sum of w_j * row when per-lookup weights are given.
 * An empty bag gives the zero vector.
 *
 *   out[b][t][d] = sum_{j in bag(t,b)} w_j * E_t[idx_j][d]        (fp64)
 *   abs_out[b][t][d] = sum_j |w_j| * |E_t[idx_j][d]|              (error scale)
 */
int oracle_emb_bag_fwd(int32_t T, int32_t D, int32_t dtype, const void *const *tables,
                       const int64_t *rows, const int64_t *indices, const int64_t *offsets,
                       const float *weights, int64_t B, double *out, double *abs_out,
                       int32_t nthreads) {
    if (T <= 0 || D <= 0 || B < 0 || !tables || !rows || !offsets || !out) return ORACLE_ERR_ARG;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
    int rc = check_csr(T, rows, indices, offsets, B);
    if (rc) return rc;
    int nt = threads_or_default(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 16)
    for (int64_t b = 0; b < B; ++b) {
        for (int t = 0; t < T; ++t) {
            int64_t bag = (int64_t)t * B + b;
            for (int d = 0; d < D; ++d) {
                double acc = 0.0, mag = 0.0;
                for (int64_t j = offsets[bag]; j < offsets[bag + 1]; ++j) {
                    double w = weights ? (double)weights[j] : 1.0;
                    double e = table_value(tables[t], dtype, indices[j], D, d);
                    acc += w * e;
                    mag += fabs(w) * fabs(e);
                }
                out[(b * T + t) * D + d] = acc;
                if (abs_out) abs_out[(b * T + t) * D + d] = mag;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Row i of the per-sample matrix X (N x D): row 0 is the dense (bottom-MLP)
 * vector, rows 1..N-1 are the pooled embeddings in table order ([P5] stage 3
 * and the interaction paragraph list the bottom-MLP output first).
 */
static double x_value(const float *dense, const float *pooled, int64_t b, int N, int D, int i,
                      int d) {
    if (i == 0) return (double)dense[b * D + d];
    return (double)pooled[(b * (int64_t)(N - 1) + (i - 1)) * D + d];
}

/*
 * Dot-product interaction, forward ([P5] stage 3 and the interaction
 * paragraph; [P2] "The architecture"; [P4]).  For the N vectors of one sample
 * take all pairwise dot products (an N x N matrix) and keep its strict upper
 * triangle, N(N-1)/2 values; then append the dense vector ([P5] stage 4: the
 * interaction values come first, then the bottom-MLP output).
 *
 * Reading: the upper-triangle values are listed row by row (i ascending, then
 * j ascending, i < j).
 *
 *   out[b] = [ <x_0,x_1>, <x_0,x_2>, ..., <x_{N-2},x_{N-1}>, dense_b[0..D-1] ]
 *   abs_out[b][p] = sum_d |x_i[d]| |x_j[d]|   (the dense part: |dense|)
 */
int oracle_interact_fwd(const float *dense, const float *pooled, int64_t B, int32_t N, int32_t D,
                        double *out, double *abs_out, int32_t nthreads) {
    if (!dense || (!pooled && N > 1) || !out || B < 0 || N < 1 || D <= 0) return ORACLE_ERR_ARG;
    int64_t P = (int64_t)N * (N - 1) / 2;
    int64_t W = P + D;
    int nt = threads_or_default(nthreads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 16)
    for (int64_t b = 0; b < B; ++b) {
        int64_t p = 0;
        for (int i = 0; i < N; ++i) {
            for (int j = i + 1; j < N; ++j) {
                double z = 0.0, mag = 0.0;
                for (int d = 0; d < D; ++d) {
                    double xi = x_value(dense, pooled, b, N, D, i, d);
                    double xj = x_value(dense, pooled, b, N, D, j, d);
                    z += xi * xj;
                    mag += fabs(xi) * fabs(xj);
                }
                out[b * W + p] = z;
                if (abs_out) abs_out[b * W + p] = mag;
                ++p;
            }
        }
        for (int d = 0; d < D; ++d) {
            out[b * W + P + d] = (double)dense[b * D + d];
            if (abs_out) abs_out[b * W + P + d] = fabs((double)dense[b * D + d]);
        }
    }
    return ORACLE_OK;
}

/*
 * Lookup fused with the interaction: the stages (2)-(4) of [P5] "Forward pass"
 * applied in sequence to one sample, the pooled vectors going straight into the
 * pairwise dots.  The value is the definition of the two stages composed; the
 * pooled rows are kept in fp64 (no rounding between the stages).
 *
 *   x_0 = dense_b,  x_{t+1}[d] = sum_{j in bag(t,b)} w_j * E_t[idx_j][d]
 *   out[b] = [ <x_i,x_j> for i < j row by row, dense_b[0..D-1] ]
 *   abs_out[b][p] = sum_d a_i[d] * a_j[d], with a_0 = |dense_b| and
 *                   a_{t+1}[d] = sum_j |w_j| |E_t[idx_j][d]|
 *
 * abs_out is the sum of the absolute values of every product w_k E_k[d] w_l E_l[d]
 * the dot expands into; the dense part of abs_out is |dense|.
 */
int oracle_emb_interact_fwd(int32_t T, int32_t D, int32_t dtype, const void *const *tables,
                            const int64_t *rows, const int64_t *indices, const int64_t *offsets,
                            const float *weights, int64_t B, const float *dense, double *out,
                            double *abs_out, int32_t nthreads) {
    if (T <= 0 || D <= 0 || B < 0 || !tables || !rows || !offsets || !dense || !out)
        return ORACLE_ERR_ARG;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_ERR_ARG;
    int rc = check_csr(T, rows, indices, offsets, B);
    if (rc) return rc;
    const int N = T + 1;
    const int64_t P = (int64_t)N * (N - 1) / 2, W = P + D;
    int nt = threads_or_default(nthreads);
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double *x = malloc(sizeof(double) * (size_t)N * D);
        double *a = malloc(sizeof(double) * (size_t)N * D);
        if (!x || !a) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t b = 0; b < B; ++b) {
            if (!x || !a) continue;
            for (int d = 0; d < D; ++d) {
                x[d] = (double)dense[b * D + d];
                a[d] = fabs(x[d]);
            }
            for (int t = 0; t < T; ++t) {
                int64_t bag = (int64_t)t * B + b;
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0, mag = 0.0;
                    for (int64_t j = offsets[bag]; j < offsets[bag + 1]; ++j) {
                        double w = weights ? (double)weights[j] : 1.0;
                        double e = table_value(tables[t], dtype, indices[j], D, d);
                        acc += w * e;
                        mag += fabs(w) * fabs(e);
                    }
                    x[(int64_t)(t + 1) * D + d] = acc;
                    a[(int64_t)(t + 1) * D + d] = mag;
                }
            }
            int64_t p = 0;
            for (int i = 0; i < N; ++i) {
                for (int j = i + 1; j < N; ++j) {
                    double z = 0.0, mag = 0.0;
                    for (int d = 0; d < D; ++d) {
                        z += x[(int64_t)i * D + d] * x[(int64_t)j * D + d];
                        mag += a[(int64_t)i * D + d] * a[(int64_t)j * D + d];
                    }
                    out[b * W + p] = z;
                    if (abs_out) abs_out[b * W + p] = mag;
                    ++p;
                }
            }
            for (int d = 0; d < D; ++d) {
                out[b * W + P + d] = x[d];
                if (abs_out) abs_out[b * W + P + d] = a[d];
            }
        }
        free(x);
        free(a);
    }
    return failed ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * Dot-product interaction, backward.  The pages give only the forward map and
 * say training runs gradient descent on it ([P5] training sentence), so this
 * is its derivative: with g the upstream gradient of out[b],
 *
 *   G[i][j] = G[j][i] = g[p(i,j)] for i < j (p: the row-major triu position),
 *   G[i][i] = 0,
 *   dX[i][d] = sum_{j != i} G[i][j] * x_j[d],
 *   grad_dense[b][d]     = dX[0][d] + g[P + d]      (the appended copy)
 *   grad_pooled[b][t][d] = dX[t+1][d].
 *
 * abs outputs: sum_{j != i} |G[i][j]| |x_j[d]| (+ |g[P+d]| for row 0).
 */
int oracle_interact_bwd(const float *grad_out, const float *dense, const float *pooled, int64_t B,
                        int32_t N, int32_t D, double *grad_dense, double *grad_pooled,
                        double *abs_dense, double *abs_pooled, int32_t nthreads) {
    if (!grad_out || !dense || !grad_dense || B < 0 || N < 1 || D <= 0) return ORACLE_ERR_ARG;
    if (N > 1 && (!pooled || !grad_pooled)) return ORACLE_ERR_ARG;
    int64_t P = (int64_t)N * (N - 1) / 2;
    int64_t W = P + D;
    int nt = threads_or_default(nthreads);
    int rc = ORACLE_OK;
#pragma omp parallel num_threads(nt)
    {
        double *G = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
        if (!G) {
#pragma omp atomic write
            rc = ORACLE_ERR_NOMEM;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t b = 0; b < B; ++b) {
            if (!G) continue;
            const float *g = grad_out + b * W;
            int64_t p = 0;
            for (int i = 0; i < N; ++i) {
                G[(int64_t)i * N + i] = 0.0;
                for (int j = i + 1; j < N; ++j) {
                    G[(int64_t)i * N + j] = (double)g[p];
                    G[(int64_t)j * N + i] = (double)g[p];
                    ++p;
                }
            }
            for (int i = 0; i < N; ++i) {
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0, mag = 0.0;
                    for (int j = 0; j < N; ++j) {
                        if (j == i) continue;
                        double gij = G[(int64_t)i * N + j];
                        double xj = x_value(dense, pooled, b, N, D, j, d);
                        acc += gij * xj;
                        mag += fabs(gij) * fabs(xj);
                    }
                    if (i == 0) {
                        acc += (double)g[P + d];
                        mag += fabs((double)g[P + d]);
                        grad_dense[b * D + d] = acc;
                        if (abs_dense) abs_dense[b * D + d] = mag;
                    } else {
                        int64_t o = (b * (int64_t)(N - 1) + (i - 1)) * D + d;
                        grad_pooled[o] = acc;
                        if (abs_pooled) abs_pooled[o] = mag;
                    }
                }
            }
        }
        free(G);
    }
    return rc;
}

typedef struct {
    int64_t key;
    int64_t pos;
} key_pos;

/* Ties are ordered by original position, so sorting (key, pos) pairs is the
 * stable sort of the keys. */
static int cmp_key_pos(const void *a, const void *b) {
    const key_pos *x = (const key_pos *)a, *y = (const key_pos *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

/*
 * Gradients of the looked-up rows, shared by the two update rules below ([P5]
 * training sentence: training uses SGD/Adagrad).  The lookup is linear in the
 * table, so the gradient of a table row is the sum, over every lookup of that
 * row, of the lookup's weight times the pooled gradient of the lookup's bag.
 *
 * Readings (the pages say nothing more):
 *   - A row's key is rowbase[t] + idx, rowbase the exclusive prefix sum of
 *     V_t.  Lookups are stably sorted by key; perm[k] is the original position
 *     of sorted position k.  unique_keys ascend; seg_offsets[u] is the first
 *     sorted position of key u and seg_offsets[U] = nnz.
 *   - G_u[d] = sum over the segment, in ascending sorted position, of
 *     w * grad_pooled[b][t][d] (fp64).
 *   - Only rows that appear are updated; each appears once in the output.
 *
 * On success *G_out holds U x D fp64 gradients (caller frees), *t_out and
 * *r_out the table and row of each unique key.
 */
typedef struct {
    int64_t U;
    double *G;   /* [U][D] */
    int32_t *t;  /* [U] */
    int64_t *r;  /* [U] */
} row_grads;

static void free_row_grads(row_grads *g) {
    free(g->G), free(g->t), free(g->r);
    g->G = NULL, g->t = NULL, g->r = NULL;
}

static int gather_row_grads(int32_t T, int32_t D, const int64_t *rows, const int64_t *indices,
                            const int64_t *offsets, const float *weights, int64_t B, int64_t nnz,
                            const float *grad_pooled, int64_t *unique_keys, int64_t *seg_offsets,
                            int32_t *perm, int64_t *num_unique, row_grads *out) {
    out->G = NULL, out->t = NULL, out->r = NULL, out->U = 0;
    if (offsets[(int64_t)T * B] != nnz) return ORACLE_ERR_OFFSETS;
    int rc = check_csr(T, rows, indices, offsets, B);
    if (rc) return rc;
    size_t n1 = (size_t)(nnz > 0 ? nnz : 1);
    int64_t *rowbase = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T + 1));
    int64_t *bag_of = (int64_t *)malloc(sizeof(int64_t) * n1);
    key_pos *kp = (key_pos *)malloc(sizeof(key_pos) * n1);
    if (!rowbase || !bag_of || !kp) {
        free(rowbase), free(bag_of), free(kp);
        return ORACLE_ERR_NOMEM;
    }
    rowbase[0] = 0;
    for (int t = 0; t < T; ++t) rowbase[t + 1] = rowbase[t] + rows[t];

    for (int64_t g = 0; g < (int64_t)T * B; ++g) {
        int64_t t = g / B;
        for (int64_t j = offsets[g]; j < offsets[g + 1]; ++j) {
            bag_of[j] = g;
            kp[j].key = rowbase[t] + indices[j];
            kp[j].pos = j;
        }
    }
    qsort(kp, (size_t)nnz, sizeof(key_pos), cmp_key_pos);
    for (int64_t k = 0; k < nnz; ++k) perm[k] = (int32_t)kp[k].pos;

    int64_t U = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        if (k == 0 || kp[k].key != kp[k - 1].key) {
            unique_keys[U] = kp[k].key;
            seg_offsets[U] = k;
            ++U;
        }
    }
    seg_offsets[U] = nnz;
    *num_unique = U;

    out->U = U;
    out->G = (double *)calloc((size_t)(U > 0 ? U : 1) * (size_t)D, sizeof(double));
    out->t = (int32_t *)malloc(sizeof(int32_t) * (size_t)(U > 0 ? U : 1));
    out->r = (int64_t *)malloc(sizeof(int64_t) * (size_t)(U > 0 ? U : 1));
    if (!out->G || !out->t || !out->r) {
        free_row_grads(out);
        free(rowbase), free(bag_of), free(kp);
        return ORACLE_ERR_NOMEM;
    }
    for (int64_t u = 0; u < U; ++u) {
        int64_t key = unique_keys[u];
        int t = 0;
        while (!(rowbase[t] <= key && key < rowbase[t + 1])) ++t;
        out->t[u] = t;
        out->r[u] = key - rowbase[t];
        double *G = out->G + u * (int64_t)D;
        for (int64_t k = seg_offsets[u]; k < seg_offsets[u + 1]; ++k) {
            int64_t j = kp[k].pos;
            int64_t b = bag_of[j] % B;
            double w = weights ? (double)weights[j] : 1.0;
            for (int d = 0; d < D; ++d) G[d] += w * (double)grad_pooled[(b * T + t) * (int64_t)D + d];
        }
    }
    free(rowbase), free(bag_of), free(kp);
    return ORACLE_OK;
}

/*
 * Embedding backward with row-wise Adagrad: the row gradients above, then one
 * accumulator per row, updated before the step:
 *         s <- s + (1/D) sum_d G_u[d]^2
 *         E[r][d] <- E[r][d] - lr * G_u[d] / (sqrt(s) + eps)
 * (Duchi, Hazan & Singer 2011 with the accumulator shared by the row).
 *
 * Outputs are per unique row u (row = unique_keys[u] - rowbase[t]):
 * new_rows[u][d] and new_state[u] in fp64.  The inputs are not modified.
 * Arrays are sized by nnz; only the first U entries (U+1 for seg_offsets) are
 * written.
 */
int oracle_emb_bag_bwd_adagrad(int32_t T, int32_t D, int32_t dtype, const void *const *tables,
                               const float *const *states, const int64_t *rows,
                               const int64_t *indices, const int64_t *offsets, const float *weights,
                               int64_t B, int64_t nnz, const float *grad_pooled, float lr, float eps,
                               int64_t *unique_keys, int64_t *seg_offsets, int32_t *perm,
                               int64_t *num_unique, double *new_rows, double *new_state) {
    if (T <= 0 || D <= 0 || B < 0 || nnz < 0 || !tables || !states || !rows || !offsets ||
        !unique_keys || !seg_offsets || !perm || !num_unique || !new_rows || !new_state)
        return ORACLE_ERR_ARG;
    if (nnz > 0 && (!indices || !grad_pooled)) return ORACLE_ERR_ARG;
    row_grads g;
    int rc = gather_row_grads(T, D, rows, indices, offsets, weights, B, nnz, grad_pooled, unique_keys,
                              seg_offsets, perm, num_unique, &g);
    if (rc) return rc;
    for (int64_t u = 0; u < g.U; ++u) {
        const double *G = g.G + u * (int64_t)D;
        int t = g.t[u];
        int64_t r = g.r[u];
        double m = 0.0;
        for (int d = 0; d < D; ++d) m += G[d] * G[d];
        m /= (double)D;
        double s = (double)states[t][r] + m;
        new_state[u] = s;
        double denom = sqrt(s) + (double)eps;
        for (int d = 0; d < D; ++d)
            new_rows[u * (int64_t)D + d] = table_value(tables[t], dtype, r, D, d) - (double)lr * G[d] / denom;
    }
    free_row_grads(&g);
    return ORACLE_OK;
}

/*
 * Embedding backward with plain SGD ([P5] training sentence names SGD): the
 * row gradients above, then for each unique row
 *         E[r][d] <- E[r][d] - lr * G_u[d]
 * Outputs as for Adagrad (no state).
 */
int oracle_emb_bag_bwd_sgd(int32_t T, int32_t D, int32_t dtype, const void *const *tables,
                           const int64_t *rows, const int64_t *indices, const int64_t *offsets,
                           const float *weights, int64_t B, int64_t nnz, const float *grad_pooled,
                           float lr, int64_t *unique_keys, int64_t *seg_offsets, int32_t *perm,
                           int64_t *num_unique, double *new_rows) {
    if (T <= 0 || D <= 0 || B < 0 || nnz < 0 || !tables || !rows || !offsets || !unique_keys ||
        !seg_offsets || !perm || !num_unique || !new_rows)
        return ORACLE_ERR_ARG;
    if (nnz > 0 && (!indices || !grad_pooled)) return ORACLE_ERR_ARG;
    row_grads g;
    int rc = gather_row_grads(T, D, rows, indices, offsets, weights, B, nnz, grad_pooled, unique_keys,
                              seg_offsets, perm, num_unique, &g);
    if (rc) return rc;
    for (int64_t u = 0; u < g.U; ++u) {
        const double *G = g.G + u * (int64_t)D;
        for (int d = 0; d < D; ++d)
            new_rows[u * (int64_t)D + d] = table_value(tables[g.t[u]], dtype, g.r[u], D, d) - (double)lr * G[d];
    }
    free_row_grads(&g);
    return ORACLE_OK;
}
