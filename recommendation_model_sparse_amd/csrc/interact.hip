// Dot-product feature interaction, forward and backward (robocikowo.com "DLRM", paragraph
// "Forward pass", stages (3)-(4), and its paragraph on the interaction layer;
// notes.helloworld.co.in "Deep Learning Recommendation Model (DLRM)", "The architecture").
//
// Per sample, X is N x D (row 0 the dense vector, rows 1..N-1 the pooled embeddings).
// Forward: the strict upper triangle of X X^T, row by row, then the dense vector.
// Backward: dX = G X with G the symmetric matrix of the upstream triu gradients.
//
// Forward on gfx950: the per-sample Gram X X^T is a dense contraction, so it runs on the matrix
// cores: v_mfma_f32_16x16x4_f32 (full fp32) over 16-row blocks of X, computing only the
// blocks on or above the diagonal.  Each lane loads its A/B operands straight from global
// memory with 16-byte loads (the k order inside a chunk is permuted identically for both
// operands, which leaves every dot product's set of terms unchanged), so no LDS is needed and
// one wavefront handles one sample, or at D = 128 and N <= 32 up to four in turn with the next
// chunk's loads in flight during the matrix-core work.  A plain-VALU kernel serves shapes the
// MFMA tiling does not cover (D not a multiple of 16).
//
// Backward: one wavefront per (sample, 128-column slice); the lane owns one or two columns d of
// X in registers, G sits in LDS and is read with broadcast loads, and dX[i][d] = sum_j G[i][j]
// X[j][d] is a register FMA chain.  Reads X once and writes dX once: HBM-bound.
#include "common.h"
#include "gram.h"

namespace dlrm {
namespace {

__device__ __forceinline__ const float *x_row(const float *dense, const float *pooled, uint32_t b,
                                              int N, int D, int i) {
    return i == 0 ? dense + static_cast<uint64_t>(b) * D
                  : pooled + (static_cast<uint64_t>(b) * (N - 1) + (i - 1)) * D;
}

// NB = ceil(N/16) row blocks; KC = k-chunk width (16 or 32); NCH = D / KC chunks; CHG = chunks
// whose operands are loaded together.
template <int NB, int KC, int NCH, int CHG>
__global__ __launch_bounds__(256) void k_interact_fwd_mfma(const float *__restrict__ dense,
                                                           const float *__restrict__ pooled,
                                                           float *__restrict__ out, uint32_t B,
                                                           int N, int P) {
    constexpr int D = KC * NCH;
    constexpr int PL = KC / 4;  // floats per lane per chunk
    constexpr int NBLK = NB * (NB + 1) / 2;
    const uint32_t sample = blockIdx.x * 4 + wave_id();
    if (sample >= B) return;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, q = lane >> 4;

    const float *rowp[NB];
    bool rv[NB];
#pragma unroll
    for (int R = 0; R < NB; ++R) {
        const int i = R * 16 + r16;
        rv[R] = i < N;
        rowp[R] = x_row(dense, pooled, sample, N, D, rv[R] ? i : 0) + q * PL;
    }
    floatx4 acc[NBLK];
#pragma unroll
    for (int k = 0; k < NBLK; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
    // the dense vector for the concatenated tail, loaded with the operands (a load at the end
    // would add a round trip to every sample)
    constexpr int DPL = (D + kWave - 1) / kWave;
    const float *dsrc = dense + static_cast<uint64_t>(sample) * D;
    float dv[DPL];
#pragma unroll
    for (int s = 0; s < DPL; ++s) dv[s] = dsrc[min(lane + s * kWave, D - 1)];

#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += CHG) {
        float x[NB][CHG][PL];
#pragma unroll
        for (int R = 0; R < NB; ++R)
#pragma unroll
            for (int c = 0; c < CHG; ++c)
#pragma unroll
                for (int v = 0; v < PL; v += 4) {
                    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (rv[R]) f = *reinterpret_cast<const float4 *>(rowp[R] + (c0 + c) * KC + v);
                    x[R][c][v] = f.x;
                    x[R][c][v + 1] = f.y;
                    x[R][c][v + 2] = f.z;
                    x[R][c][v + 3] = f.w;
                }
#pragma unroll
        for (int c = 0; c < CHG; ++c)
#pragma unroll
            for (int s = 0; s < PL; ++s) {
                int k = 0;
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int J = I; J < NB; ++J, ++k)
                        acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[I][c][s], x[J][c][s],
                                                                      acc[k], 0, 0, 0);
            }
    }
    // D[i][j] of block (I,J) sits in lane j + 16*(i/4), element i%4
    float *orow = out + static_cast<uint64_t>(sample) * (P + D);
    int k = 0;
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int J = I; J < NB; ++J, ++k)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int gi = I * 16 + q * 4 + v, gj = J * 16 + r16;
                if (gi < gj && gj < N) orow[triu_pos(gi, gj, N)] = acc[k][v];
            }
#pragma unroll
    for (int s = 0; s < DPL; ++s)
        if (lane + s * kWave < D) orow[P + lane + s * kWave] = dv[s];
}

// The same Gram as k_interact_fwd_mfma, SPW samples per wavefront in turn, one k-chunk of
// operands in registers and the next one in flight: the loads of chunk c+1 (or of the next
// sample's first chunk and dense vector) are issued before the matrix-core work of chunk c.
template <int NB, int KC, int NCH, int SPW>
__global__ __launch_bounds__(256) void k_interact_fwd_mfma_pipe(const float *__restrict__ dense,
                                                                const float *__restrict__ pooled,
                                                                float *__restrict__ out, uint32_t B,
                                                                int N, int P) {
    constexpr int D = KC * NCH;
    constexpr int PL = KC / 4;
    constexpr int NBLK = NB * (NB + 1) / 2;
    constexpr int DPL = (D + kWave - 1) / kWave;
    const uint32_t s0 = (blockIdx.x * 4 + wave_id()) * SPW;
    if (s0 >= B) return;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, q = lane >> 4;
    bool rv[NB];
    int ri[NB];
#pragma unroll
    for (int R = 0; R < NB; ++R) {
        const int i = R * 16 + r16;
        rv[R] = i < N;
        ri[R] = rv[R] ? i : 0;
    }
    auto load_chunk = [&](uint32_t sample, int c, float (&x)[NB][PL]) {
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            const float *p = x_row(dense, pooled, sample, N, D, ri[R]) + q * PL + c * KC;
#pragma unroll
            for (int v = 0; v < PL; v += 4) {
                float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
                if (rv[R]) f = *reinterpret_cast<const float4 *>(p + v);
                x[R][v] = f.x, x[R][v + 1] = f.y, x[R][v + 2] = f.z, x[R][v + 3] = f.w;
            }
        }
    };
    auto load_dense = [&](uint32_t sample, float (&dv)[DPL]) {
        const float *dsrc = dense + static_cast<uint64_t>(sample) * D;
#pragma unroll
        for (int s = 0; s < DPL; ++s) dv[s] = dsrc[min(lane + s * kWave, D - 1)];
    };
    float x[NB][PL], dv[DPL];
    load_dense(s0, dv);
    load_chunk(s0, 0, x);
#pragma unroll
    for (int si = 0; si < SPW; ++si) {
        const uint32_t sample = s0 + si;
        if (sample >= B) break;  // wave-uniform
        const uint32_t next = min(sample + 1, B - 1);
        floatx4 acc[NBLK];
#pragma unroll
        for (int k = 0; k < NBLK; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
        float dn[DPL];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            float xn[NB][PL];
            if (c + 1 < NCH) load_chunk(sample, c + 1, xn);
            else if (si + 1 < SPW) {
                load_dense(next, dn);
                load_chunk(next, 0, xn);
            }
#pragma unroll
            for (int s = 0; s < PL; ++s) {
                int k = 0;
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int J = I; J < NB; ++J, ++k)
                        acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[I][s], x[J][s], acc[k], 0, 0, 0);
            }
            if (c + 1 < NCH || si + 1 < SPW) {
#pragma unroll
                for (int R = 0; R < NB; ++R)
#pragma unroll
                    for (int v = 0; v < PL; ++v) x[R][v] = xn[R][v];
            }
        }
        float *orow = out + static_cast<uint64_t>(sample) * (P + D);
        int k = 0;
#pragma unroll
        for (int I = 0; I < NB; ++I)
#pragma unroll
            for (int J = I; J < NB; ++J, ++k)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int gi = I * 16 + q * 4 + v, gj = J * 16 + r16;
                    if (gi < gj && gj < N) orow[triu_pos(gi, gj, N)] = acc[k][v];
                }
#pragma unroll
        for (int s = 0; s < DPL; ++s)
            if (lane + s * kWave < D) orow[P + lane + s * kWave] = dv[s];
        if (si + 1 < SPW) {
#pragma unroll
            for (int s = 0; s < DPL; ++s) dv[s] = dn[s];
        }
    }
}

// Any D % 4 == 0: one block per sample, one thread per pair, fp32 FMA chain over d.
__global__ __launch_bounds__(256) void k_interact_fwd_valu(const float *__restrict__ dense,
                                                           const float *__restrict__ pooled,
                                                           float *__restrict__ out, int N, int D,
                                                           int P) {
    const uint32_t sample = blockIdx.x;
    float *orow = out + static_cast<uint64_t>(sample) * (P + D);
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        // invert the row-major triu position
        int i = 0, rem = p;
        while (rem >= N - 1 - i) {
            rem -= N - 1 - i;
            ++i;
        }
        const int j = i + 1 + rem;
        const float *xi = x_row(dense, pooled, sample, N, D, i);
        const float *xj = x_row(dense, pooled, sample, N, D, j);
        float z = 0.f;
        for (int d = 0; d < D; d += 4) {
            const float4 a = *reinterpret_cast<const float4 *>(xi + d);
            const float4 b = *reinterpret_cast<const float4 *>(xj + d);
            z = fmaf(a.x, b.x, z);
            z = fmaf(a.y, b.y, z);
            z = fmaf(a.z, b.z, z);
            z = fmaf(a.w, b.w, z);
        }
        orow[p] = z;
    }
    const float *dsrc = dense + static_cast<uint64_t>(sample) * D;
    for (int d = threadIdx.x; d < D; d += blockDim.x) orow[P + d] = dsrc[d];
}

// The plain-VALU contender of the matrix-core Gram (selected by dlrm_interact_fwd_ex): the X of S
// samples staged in LDS with contiguous 16-byte loads, rows padded by 4 floats; each thread then
// computes a TILE x TILE block of dots of one sample, an FMA chain over d in order, with its
// 2*TILE operand rows read from LDS.  Blocks (I, J) with I <= J cover the upper triangle.
template <int TILE>
__global__ __launch_bounds__(256) void k_interact_fwd_lds(const float *__restrict__ dense,
                                                          const float *__restrict__ pooled,
                                                          float *__restrict__ out, uint32_t B, int N, int D,
                                                          int P, int S) {
    extern __shared__ float xs[];  // [S][N][D + 4]
    const int LD = D + 4, D4 = D / 4;
    const uint32_t b0 = blockIdx.x * S;
    const int ns = static_cast<int>(min(static_cast<uint32_t>(S), B - b0));
    for (int q = threadIdx.x; q < ns * N * D4; q += blockDim.x) {
        const int sm = q / (N * D4), rem = q - sm * (N * D4), i = rem / D4, d4 = rem - i * D4;
        const float4 v = *reinterpret_cast<const float4 *>(x_row(dense, pooled, b0 + sm, N, D, i) + d4 * 4);
        *reinterpret_cast<float4 *>(xs + (sm * N + i) * LD + d4 * 4) = v;
    }
    __syncthreads();
    const int NT = (N + TILE - 1) / TILE;
    const int tiles = NT * (NT + 1) / 2;
    for (int q = threadIdx.x; q < ns * tiles; q += blockDim.x) {
        const int sm = q / tiles;
        int t = q - sm * tiles, I = 0;
        while (t >= NT - I) t -= NT - I, ++I;
        const int J = I + t;
        const float *xi = xs + (sm * N + I * TILE) * LD, *xj = xs + (sm * N + J * TILE) * LD;
        float acc[TILE][TILE];
#pragma unroll
        for (int a = 0; a < TILE; ++a)
#pragma unroll
            for (int c = 0; c < TILE; ++c) acc[a][c] = 0.f;
        for (int d = 0; d < D; d += 4) {
            float4 u[TILE], v[TILE];
#pragma unroll
            for (int a = 0; a < TILE; ++a) {  // rows past N read row N-1's slot and are never stored
                u[a] = *reinterpret_cast<const float4 *>(xi + min(a, N - 1 - I * TILE) * LD + d);
                v[a] = *reinterpret_cast<const float4 *>(xj + min(a, N - 1 - J * TILE) * LD + d);
            }
#pragma unroll
            for (int a = 0; a < TILE; ++a)
#pragma unroll
                for (int c = 0; c < TILE; ++c) {
                    acc[a][c] = fmaf(u[a].x, v[c].x, acc[a][c]);
                    acc[a][c] = fmaf(u[a].y, v[c].y, acc[a][c]);
                    acc[a][c] = fmaf(u[a].z, v[c].z, acc[a][c]);
                    acc[a][c] = fmaf(u[a].w, v[c].w, acc[a][c]);
                }
        }
        float *orow = out + static_cast<uint64_t>(b0 + sm) * (P + D);
#pragma unroll
        for (int a = 0; a < TILE; ++a)
#pragma unroll
            for (int c = 0; c < TILE; ++c) {
                const int i = I * TILE + a, j = J * TILE + c;
                if (i < j && j < N) orow[triu_pos(i, j, N)] = acc[a][c];
            }
    }
    // the dense vector after the dots
    for (int q = threadIdx.x; q < ns * D; q += blockDim.x) {
        const int sm = q / D, d = q - sm * D;
        out[static_cast<uint64_t>(b0 + sm) * (P + D) + P + d] = xs[sm * N * LD + d];
    }
}

// Small interactions (N <= 11, D = 64 * CPL): the k-split Gram (gram.h) over NR = gram_rows(N)
// rows, M samples per wave.  Lane l loads columns l*CPL.. of every row (each row read is one
// coalesced load), and every load is unconditional (rows past N re-read row N-1 and are zeroed)
// so all are in flight at once.
template <int NR, int CPL, int M>
__global__ __launch_bounds__(256) void k_interact_fwd_ksplit(const float *__restrict__ dense,
                                                             const float *__restrict__ pooled,
                                                             float *__restrict__ out, uint32_t B,
                                                             int N, int P) {
    constexpr int D = 64 * CPL;
    const uint32_t b0 = (blockIdx.x * 4 + wave_id()) * M;
    if (b0 >= B) return;
    const int lane = threadIdx.x & 63;
    float x[M][NR][CPL];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t b = min(b0 + m, B - 1);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int ii = i < N ? i : N - 1;
            uint32_t w[CPL];
            gload_words<CPL>(x_row(dense, pooled, b, N, D, ii) + lane * CPL, w);
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[m][i][c] = i < N ? __uint_as_float(w[c]) : 0.f;
        }
    }
    int pi, pj;
    const bool holds = gram_lane_pair<NR>(lane, pi, pj);
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t b = b0 + m;
        if (b >= B) break;  // wave-uniform
        const float z = gram_ksplit<NR, CPL>(x[m]);
        float *orow = out + static_cast<uint64_t>(b) * (P + D);
        if (holds && pj < N) orow[triu_pos(pi, pj, N)] = z;
#pragma unroll
        for (int c = 0; c < CPL; ++c) orow[P + lane * CPL + c] = x[m][0][c];
    }
}

// Backward.  NP = padded N (multiple of 4, >= N); CPL = columns per lane (1 or 2).
template <int NP, int CPL>
__global__ __launch_bounds__(256) void k_interact_bwd(const float *__restrict__ grad_out,
                                                      const float *__restrict__ dense,
                                                      const float *__restrict__ pooled,
                                                      float *__restrict__ grad_dense,
                                                      float *__restrict__ grad_pooled, uint32_t B,
                                                      int N, int D, int P, int slices) {
    __shared__ float Gs[4][NP][NP];
    const int wv = static_cast<int>(wave_id()), lane = threadIdx.x & 63;
    const uint64_t gw = static_cast<uint64_t>(blockIdx.x) * 4 + wv;
    const uint32_t sample = static_cast<uint32_t>(gw / slices);
    const int slice = static_cast<int>(gw % slices);
    const bool valid = sample < B;
    const uint32_t sb = valid ? sample : 0;
    const float *g = grad_out + static_cast<uint64_t>(sb) * (P + D);

    // this lane's columns of X and of the dense part of the upstream gradient are loaded first,
    // so that their round trip overlaps the one of the G loads below
    const int d0 = slice * (kWave * CPL) + lane * CPL;
    const bool dv = valid && d0 < D;
    float gt[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) gt[c] = dv ? g[P + d0 + c] : 0.f;
    float x[NP][CPL];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        if (dv && j < N) {
            const float *src = x_row(dense, pooled, sb, N, D, j) + d0;
            if constexpr (CPL == 2) {
                const float2 f = *reinterpret_cast<const float2 *>(src);
                x[j][0] = f.x;
                x[j][1] = f.y;
            } else {
                x[j][0] = src[0];
            }
        } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[j][c] = 0.f;
        }
    }
    // G: symmetric, zero diagonal, zero padding.  All of a lane's entries are loaded before any
    // is stored (every load unconditional: entries off the triangle re-read entry 0 and are
    // zeroed), so they make one round trip rather than one per entry.
    constexpr int NE = (NP * NP + kWave - 1) / kWave;
    float gv_[NE];
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = lane + k * kWave, i = e / NP, j = e % NP;
        const bool on = valid && e < NP * NP && i < N && j < N && i != j;
        const float v = g[on ? (i < j ? triu_pos(i, j, N) : triu_pos(j, i, N)) : 0];
        gv_[k] = on ? v : 0.f;
    }
#pragma unroll
    for (int k = 0; k < NE; ++k) {
        const int e = lane + k * kWave;
        if (e < NP * NP) Gs[wv][e / NP][e % NP] = gv_[k];
    }
    __syncthreads();

    if (!dv) return;
    for (int i = 0; i < N; ++i) {
        float acc[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll
        for (int j = 0; j < NP; j += 4) {
            const float4 gv = *reinterpret_cast<const float4 *>(&Gs[wv][i][j]);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                acc[c] = fmaf(gv.x, x[j][c], acc[c]);
                acc[c] = fmaf(gv.y, x[j + 1][c], acc[c]);
                acc[c] = fmaf(gv.z, x[j + 2][c], acc[c]);
                acc[c] = fmaf(gv.w, x[j + 3][c], acc[c]);
            }
        }
        float *dst;
        if (i == 0) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] += gt[c];
            dst = grad_dense + static_cast<uint64_t>(sb) * D + d0;
        } else {
            dst = grad_pooled + (static_cast<uint64_t>(sb) * (N - 1) + (i - 1)) * D + d0;
        }
        if constexpr (CPL == 2) *reinterpret_cast<float2 *>(dst) = make_float2(acc[0], acc[1]);
        else dst[0] = acc[0];
    }
}

template <int NR>
void launch_fwd_ksplit(const float *dense, const float *pooled, float *out, uint32_t b, int N, int D, int P,
                       hipStream_t stream) {
    switch (D) {
        case 64: DLRM_LAUNCH("interact_fwd_ksplit", (k_interact_fwd_ksplit<NR, 1, 2>), dim3((b + 7) / 8), dim3(256), 0, stream, dense, pooled, out, b, N, P); break;
        case 128: DLRM_LAUNCH("interact_fwd_ksplit", (k_interact_fwd_ksplit<NR, 2, 2>), dim3((b + 7) / 8), dim3(256), 0, stream, dense, pooled, out, b, N, P); break;
        default: DLRM_LAUNCH("interact_fwd_ksplit", (k_interact_fwd_ksplit<NR, 4, 1>), dim3((b + 3) / 4), dim3(256), 0, stream, dense, pooled, out, b, N, P); break;
    }
}

template <int NB, int SPW>
void launch_fwd_pipe(const float *dense, const float *pooled, float *out, uint32_t B, int N, int P,
                     hipStream_t stream) {
    const uint32_t waves = (B + SPW - 1) / SPW;
    DLRM_LAUNCH("interact_fwd_mfma", (k_interact_fwd_mfma_pipe<NB, 32, 4, SPW>), dim3((waves + 3) / 4), dim3(256), 0,
                stream, dense, pooled, out, B, N, P);
}

template <int NB>
bool launch_fwd_mfma(const float *dense, const float *pooled, float *out, uint32_t B, int N, int D,
                     int P, hipStream_t stream) {
    const dim3 grid((B + 3) / 4), block(256);
    // operands of CHG chunks are loaded at once: NB*CHG*KC/4 registers, kept <= 64
    switch (D) {
        case 16: DLRM_LAUNCH("interact_fwd_mfma", (k_interact_fwd_mfma<NB, 16, 1, 1>), grid, block, 0, stream, dense, pooled, out, B, N, P); return true;
        case 32: DLRM_LAUNCH("interact_fwd_mfma", (k_interact_fwd_mfma<NB, 32, 1, 1>), grid, block, 0, stream, dense, pooled, out, B, N, P); return true;
        case 64: DLRM_LAUNCH("interact_fwd_mfma", (k_interact_fwd_mfma<NB, 32, 2, (NB <= 4 ? 2 : 1)>), grid, block, 0, stream, dense, pooled, out, B, N, P); return true;
        case 128:
            if constexpr (NB <= 2) {
                // samples per wavefront by batch size: enough waves to fill the chip first, then
                // longer chains of overlapped samples (16384 samples at N = 27: 55.7 us one per
                // wave, 52.1 two, 50.8 four; 4099 samples: 18.6 / 17.3 / 20.0 us)
                if (B >= 12288) launch_fwd_pipe<NB, 4>(dense, pooled, out, B, N, P, stream);
                else if (B >= 3072) launch_fwd_pipe<NB, 2>(dense, pooled, out, B, N, P, stream);
                else launch_fwd_pipe<NB, 1>(dense, pooled, out, B, N, P, stream);
                return true;
            }
            // one chunk's operands at a time (16 registers): more waves per SIMD, which beat
            // loading the whole row at once
            DLRM_LAUNCH("interact_fwd_mfma", (k_interact_fwd_mfma<NB, 32, 4, 1>), grid, block, 0, stream, dense, pooled, out, B, N, P); return true;
        case 256: DLRM_LAUNCH("interact_fwd_mfma", (k_interact_fwd_mfma<NB, 32, 8, (NB <= 2 ? 4 : (NB <= 4 ? 2 : 1))>), grid, block, 0, stream, dense, pooled, out, B, N, P); return true;
        case 512: DLRM_LAUNCH("interact_fwd_mfma", (k_interact_fwd_mfma<NB, 32, 16, (NB <= 2 ? 4 : (NB <= 4 ? 2 : 1))>), grid, block, 0, stream, dense, pooled, out, B, N, P); return true;
        default: return false;
    }
}

template <int NP>
void launch_bwd(const float *g, const float *dense, const float *pooled, float *gd, float *gp,
                uint32_t B, int N, int D, int P, hipStream_t stream) {
    if (D >= 128) {
        const int slices = (D + 127) / 128;
        const uint64_t waves = static_cast<uint64_t>(B) * slices;
        DLRM_LAUNCH("interact_bwd", (k_interact_bwd<NP, 2>), dim3((waves + 3) / 4), dim3(256), 0, stream, g,
                           dense, pooled, gd, gp, B, N, D, P, slices);
    } else {
        const int slices = (D + 63) / 64;
        const uint64_t waves = static_cast<uint64_t>(B) * slices;
        DLRM_LAUNCH("interact_bwd", (k_interact_bwd<NP, 1>), dim3((waves + 3) / 4), dim3(256), 0, stream, g,
                           dense, pooled, gd, gp, B, N, D, P, slices);
    }
}

int check_interact(const void *a, const void *b, const void *c, int64_t B, int32_t N, int32_t D) {
    if (B < 0 || N < 1 || N > kMaxTables + 1 || D < 1) return DLRM_ERR_INVALID_ARG;
    if (D > 512 || D % 4 != 0) return DLRM_ERR_UNSUPPORTED;
    if (B >= (int64_t(1) << 31) / 4) return DLRM_ERR_UNSUPPORTED;
    if (B == 0) return DLRM_OK;
    if (!a || !c || (N > 1 && !b)) return DLRM_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(c, 4) || (b && !aligned(b, 16))) return DLRM_ERR_INVALID_ARG;
    return DLRM_OK;
}

}  // namespace
}  // namespace dlrm

namespace dlrm {
namespace {

// Samples per block of the LDS kernel: enough 2x2 tiles for the block's 256 threads, within 64 KiB.
int lds_samples(int N, int D) {
    const int NT = (N + 1) / 2, tiles = NT * (NT + 1) / 2;
    const int bytes = N * (D + 4) * 4;
    int S = (256 + tiles - 1) / tiles;
    while (S > 1 && S * bytes > 64 * 1024) --S;
    return S;
}

int interact_fwd_impl(const float *dense, const float *pooled, int64_t B, int32_t N, int32_t D, float *out,
                      int32_t path, hipStream_t stream) {
    int rc = check_interact(dense, pooled, out, B, N, D);
    if (rc != DLRM_OK || B == 0) return rc;
    const int P = N * (N - 1) / 2;
    const uint32_t b = static_cast<uint32_t>(B);
    if (path == DLRM_GRAM_VALU) {
        if (N < 2 || D % 16 != 0 || N * (D + 4) * 4 > 64 * 1024) return DLRM_ERR_UNSUPPORTED;
        const int S = lds_samples(N, D);
        DLRM_LAUNCH("interact_fwd_lds", k_interact_fwd_lds<2>, dim3((b + S - 1) / S), dim3(256),
                    static_cast<size_t>(S) * N * (D + 4) * 4, stream, dense, pooled, out, b, N, D, P, S);
        return launch_status();
    }
    if (path == DLRM_GRAM_AUTO && gram_ksplit_ok(N, D)) {
        if (gram_rows(N) == 9) launch_fwd_ksplit<9>(dense, pooled, out, b, N, D, P, stream);
        else launch_fwd_ksplit<11>(dense, pooled, out, b, N, D, P, stream);
        return launch_status();
    }
    bool done = false;
    switch ((N + 15) / 16) {
        case 1: done = launch_fwd_mfma<1>(dense, pooled, out, b, N, D, P, stream); break;
        case 2: done = launch_fwd_mfma<2>(dense, pooled, out, b, N, D, P, stream); break;
        case 3: done = launch_fwd_mfma<3>(dense, pooled, out, b, N, D, P, stream); break;
        case 4: done = launch_fwd_mfma<4>(dense, pooled, out, b, N, D, P, stream); break;
        case 5: done = launch_fwd_mfma<5>(dense, pooled, out, b, N, D, P, stream); break;
    }
    if (!done) {
        if (path == DLRM_GRAM_MFMA) return DLRM_ERR_UNSUPPORTED;
        DLRM_LAUNCH("interact_fwd_valu", k_interact_fwd_valu, dim3(b), dim3(256), 0, stream, dense, pooled, out,
                    N, D, P);
    }
    return launch_status();
}

}  // namespace
}  // namespace dlrm

extern "C" int dlrm_interact_fwd(const float *dense, const float *pooled, int64_t B, int32_t N,
                                 int32_t D, float *out, dlrm_stream_t stream_) {
    return dlrm::interact_fwd_impl(dense, pooled, B, N, D, out, DLRM_GRAM_AUTO,
                                   reinterpret_cast<hipStream_t>(stream_));
}

extern "C" int dlrm_interact_fwd_ex(const float *dense, const float *pooled, int64_t B, int32_t N, int32_t D,
                                    float *out, int32_t path, dlrm_stream_t stream_) {
    if (path != DLRM_GRAM_AUTO && path != DLRM_GRAM_MFMA && path != DLRM_GRAM_VALU) return DLRM_ERR_INVALID_ARG;
    return dlrm::interact_fwd_impl(dense, pooled, B, N, D, out, path, reinterpret_cast<hipStream_t>(stream_));
}

extern "C" int dlrm_interact_bwd(const float *grad_out, const float *dense, const float *pooled,
                                 int64_t B, int32_t N, int32_t D, float *grad_dense,
                                 float *grad_pooled, dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc = check_interact(dense, pooled, grad_dense, B, N, D);
    if (rc != DLRM_OK || B == 0) return rc;
    if (!grad_out || !aligned(grad_out, 4) || (N > 1 && (!grad_pooled || !aligned(grad_pooled, 16))))
        return DLRM_ERR_INVALID_ARG;
    if (!aligned(grad_dense, 16)) return DLRM_ERR_INVALID_ARG;
    const int P = N * (N - 1) / 2;
    const uint32_t b = static_cast<uint32_t>(B);
    if (N <= 8) launch_bwd<8>(grad_out, dense, pooled, grad_dense, grad_pooled, b, N, D, P, stream);
    else if (N <= 16) launch_bwd<16>(grad_out, dense, pooled, grad_dense, grad_pooled, b, N, D, P, stream);
    else if (N <= 32) launch_bwd<32>(grad_out, dense, pooled, grad_dense, grad_pooled, b, N, D, P, stream);
    else if (N <= 48) launch_bwd<48>(grad_out, dense, pooled, grad_dense, grad_pooled, b, N, D, P, stream);
    else launch_bwd<68>(grad_out, dense, pooled, grad_dense, grad_pooled, b, N, D, P, stream);
    return launch_status();
}
