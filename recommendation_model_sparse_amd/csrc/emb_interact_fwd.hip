// Embedding-bag lookup fused with the dot-product interaction, for inference (robocikowo.com
// "DLRM", paragraph "Forward pass": stage (2) looks the sparse features up, stage (3) takes the
// pairwise dots of the N vectors, stage (4) concatenates them with the bottom-MLP output).
//
// The unfused path writes the pooled rows to HBM as fp32 [B][T][D] and the interaction reads
// them back; here they never leave the chip.  One block owns S samples: it stages the dense
// vectors and the bags' offsets in LDS, pools every bag of its samples straight into an LDS
// copy of X (N x D fp32 per sample, rows padded by 4 floats so the matrix-core operand reads
// hit 64 distinct banks), then computes the strict upper triangle of X X^T on the matrix cores
// and writes [triu | dense].
//
// The arithmetic is the unfused path's, step for step, so the two give identical bits:
//   - pooling: the same lane-group layout, lookup-to-group assignment, fixed butterfly and
//     kernel choice (a wavefront per bag when bags hold 4+ lookups on average, else a lane
//     group per bag, rows summed in order);
//   - Gram: v_mfma_f32_16x16x4_f32 over 16-row blocks with the same k order (k-chunks of KC
//     columns, lane quarter q taking KC/4 consecutive columns of each chunk).
// Each upper 16 x 16 block of a sample's Gram is one job for one wavefront, so the 3 blocks of
// N = 27 spread over three of the block's waves.
//
// Multi-hot bags: while a wave gathers the rows of one bag it already has the first indices of
// its next bag in flight, so a bag costs one memory latency rather than two.
#include "common.h"
#include "gram.h"
#include "pool.h"

namespace dlrm {

int check_csr_on_device(const int64_t *rows, int32_t T, const void *indices, const void *offsets,
                        int32_t index_type, int64_t B, int64_t nnz, int *flag, hipStream_t stream);

namespace {

struct FusedArgs {
    const char *tables[kMaxTables];
    const int64_t *indices;
    const int64_t *offsets;
    const float *weights;
    const float *dense;
    float *out;
    uint32_t B;
    int32_t T;          // tables; N = T + 1 vectors per sample
    int32_t N;
    int32_t P;          // N(N-1)/2
    int32_t NB;         // 16-row blocks of X: ceil(N / 16)
    int32_t NBLK;       // upper blocks: NB(NB+1)/2
    int32_t S;          // samples per block
    int32_t BPG;        // bags per lane group and pass (group-per-bag pooling)
    uint32_t row_bytes;
    int32_t ksplit;     // the Gram is the k-split one of gram.h (N <= 11, D in {64, 128, 256})
};

constexpr int kPad = 4;  // floats of padding per LDS row of X

#ifndef DLRM_FUSED_M
#define DLRM_FUSED_M 2  // samples per wave in the register path when NB * D <= 128
#endif

// Dynamic LDS: X [S][N][D + kPad] fp32, then the bags' offsets [T][S + 1] int64.
__host__ __device__ inline size_t fused_lds_bytes(int S, int N, int D, int T) {
    return static_cast<size_t>(S) * N * (D + kPad) * 4 + static_cast<size_t>(T) * (S + 1) * 8;
}

// (I, J) of upper block number kb, blocks listed row by row (I <= J).
__device__ __forceinline__ void upper_block(int kb, int NB, int &I, int &J) {
    I = 0;
    while (kb >= NB - I) {
        kb -= NB - I;
        ++I;
    }
    J = I + kb;
}

// The k-split Gram of the samples staged in LDS (X [S][N][XS]), one sample per wave at a time.
template <int NR, int CPL>
__device__ __forceinline__ void lds_ksplit(const FusedArgs &a, const float *X, int XS, int Sb, uint32_t b0, int wv,
                                           int lane) {
    const int N = a.N, W = a.P + 64 * CPL;
    int pi, pj;
    const bool holds = gram_lane_pair<NR>(lane, pi, pj);
    for (int s = wv; s < Sb; s += 4) {
        const float *xs = X + static_cast<size_t>(s) * N * XS + lane * CPL;
        float x[NR][CPL];
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c) x[i][c] = i < N ? xs[i * XS + c] : 0.f;
        const float z = gram_ksplit<NR, CPL>(x);
        if (holds && pj < N) a.out[(static_cast<uint64_t>(b0) + s) * W + triu_pos(pi, pj, N)] = z;
    }
}

// Waves per SIMD the compiler is asked to fit.  The unweighted multi-hot kernel with the
// matrix-core Gram and rows of 16+ chunks fits 8 in 64 registers with no spill, against 7 by
// default (62 VGPRs + 4 AGPRs for the MFMA accumulators at 256-byte rows); the extra wave keeps
// more row loads in flight.  With 8-chunk rows the same request spills, so those keep the default.
constexpr int fused_min_waves(int G, bool weighted, bool wpb, bool ksplit) {
    return wpb && !weighted && !ksplit && G >= 16 ? 8 : 1;
}

// KSPLIT: the Gram is the k-split one of gram.h (N <= 11, D in {64, 128, 256}), else the
// matrix-core one; a template parameter, so each kernel carries only its own Gram's registers.
template <int DT, int G, int KC, bool WEIGHTED, bool WAVE_PER_BAG, bool KSPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(fused_min_waves(G, WEIGHTED, WAVE_PER_BAG, KSPLIT))))
void k_emb_interact_fwd(FusedArgs a) {
    constexpr int EPC = Elem<DT>::kPerChunk;
    constexpr int D = G * EPC;  // G 16-byte chunks per row
    constexpr int NG = kWave / G;
    constexpr int XS = D + kPad;
    constexpr int PL = KC / 4;
    constexpr int NCH = D / KC;
    static_assert(D % KC == 0 && PL % 4 == 0, "k-chunks tile the row");
    extern __shared__ __align__(16) float smem[];

    const int S = a.S, T = a.T, N = a.N;
    const uint32_t b0 = blockIdx.x * static_cast<uint32_t>(S);
    const int Sb = static_cast<int>(min(static_cast<uint32_t>(S), a.B - b0));
    float *X = smem;
    int64_t *offs = reinterpret_cast<int64_t *>(smem + static_cast<size_t>(S) * N * XS);
    const int tid = threadIdx.x, wv = static_cast<int>(wave_id()), lane = tid & 63;

    // ---- stage the bags' offsets and the dense rows (row 0 of each X)
    for (int i = tid; i < T * (Sb + 1); i += 256) {
        const int t = i / (Sb + 1), k = i - t * (Sb + 1);
        offs[t * (S + 1) + k] = a.offsets[static_cast<uint64_t>(t) * a.B + b0 + k];
    }
    for (int i = tid; i < Sb * (D / 4); i += 256) {
        const int s = i / (D / 4), q = i - s * (D / 4);
        const float4 v = *reinterpret_cast<const float4 *>(a.dense + (static_cast<uint64_t>(b0) + s) * D + 4 * q);
        *reinterpret_cast<float4 *>(X + static_cast<size_t>(s) * N * XS + 4 * q) = v;
    }
    __syncthreads();

    // ---- pool every bag (s, t) of the block into X[s][t + 1]
    const int nbags = Sb * T;
    const int grp = lane / G, c = lane % G;
    if constexpr (WAVE_PER_BAG) {
        constexpr int U = 8;
        // first chunk of indices (and weights) of the wave's next bag, loaded one bag ahead
        int64_t nx_idx = 0;
        float nx_w = 1.f;
        auto fetch_first = [&](int k) {
            const int s = k / T, t = k - s * T;
            const int64_t st = offs[t * (S + 1) + s], en = offs[t * (S + 1) + s + 1];
            const int n = static_cast<int>(min<int64_t>(kWave, en - st));
            nx_idx = lane < n ? a.indices[st + lane] : 0;
            if constexpr (WEIGHTED) nx_w = lane < n ? a.weights[st + lane] : 0.f;
        };
        if (wv < nbags) fetch_first(wv);
        for (int k = wv; k < nbags; k += 4) {
            const int s = k / T, t = k - s * T;
            const int64_t start = offs[t * (S + 1) + s], end = offs[t * (S + 1) + s + 1];
            int64_t my_idx = nx_idx;
            float my_w = nx_w;
            if (k + 4 < nbags) fetch_first(k + 4);
            const char *tab = a.tables[t] + c * 16;
            float acc[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
            for (int64_t base = start; base < end; base += kWave) {
                const int n = static_cast<int>(min<int64_t>(kWave, end - base));
                if (base != start) {  // bags longer than 64 lookups
                    my_idx = lane < n ? a.indices[base + lane] : 0;
                    if constexpr (WEIGHTED) my_w = lane < n ? a.weights[base + lane] : 0.f;
                }
                for (int r0 = 0; r0 < n; r0 += NG * U) {
                    uint4 v[U];
                    float w[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {  // lanes past the bag load nothing (no address cycles)
                        const int r = r0 + u * NG + grp;
                        const int src = r < n ? r : 0;
                        const int64_t idx = __shfl(my_idx, src);
                        w[u] = WEIGHTED ? __shfl(my_w, src) : 1.f;
                        v[u] = r < n ? load_row_chunk(tab, idx, a.row_bytes) : make_uint4(0, 0, 0, 0);
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (r0 + u * NG + grp < n) accumulate<DT, WEIGHTED>(acc, v[u], w[u]);
                }
            }
#pragma unroll
            for (int sh = G; sh < kWave; sh <<= 1)
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], sh);
            if (grp == 0) {
                float *dst = X + (static_cast<size_t>(s) * N + t + 1) * XS + c * EPC;
#pragma unroll
                for (int e = 0; e < EPC; e += 4)
                    *reinterpret_cast<float4 *>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
            }
        }
    } else {
        // a lane group per bag: worker g takes bags g, g + 4*NG, ...; BPG first rows in flight
        constexpr int MAXB = 4;
        const int worker = wv * NG + grp, nworkers = 4 * NG;
        for (int k0 = worker; k0 < nbags; k0 += nworkers * a.BPG) {
            for (int kb = 0; kb < a.BPG; kb += MAXB) {
                int64_t st[MAXB], en[MAXB];
                const char *tab[MAXB];
                int ss[MAXB], tt[MAXB];
#pragma unroll
                for (int m = 0; m < MAXB; ++m) {
                    const int k = k0 + (kb + m) * nworkers;
                    const bool ok = kb + m < a.BPG && k < nbags;
                    const int s = ok ? k / T : 0, t = ok ? k - s * T : 0;
                    ss[m] = s;
                    tt[m] = t;
                    st[m] = ok ? offs[t * (S + 1) + s] : 0;
                    en[m] = ok ? offs[t * (S + 1) + s + 1] : -1;  // -1: no bag
                    tab[m] = a.tables[t] + c * 16;
                }
                float acc[MAXB][EPC];
#pragma unroll
                for (int m = 0; m < MAXB; ++m)
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc[m][e] = 0.f;
                {
                    int64_t idx[MAXB];
                    float w[MAXB];
#pragma unroll
                    for (int m = 0; m < MAXB; ++m) {
                        const bool has = st[m] < en[m];
                        idx[m] = has ? a.indices[st[m]] : 0;
                        w[m] = (WEIGHTED && has) ? a.weights[st[m]] : 1.f;
                    }
                    uint4 v[MAXB];
#pragma unroll
                    for (int m = 0; m < MAXB; ++m) v[m] = load_row_chunk(tab[m], idx[m], a.row_bytes);
#pragma unroll
                    for (int m = 0; m < MAXB; ++m)
                        if (st[m] < en[m]) accumulate<DT, WEIGHTED>(acc[m], v[m], w[m]);
                }
#pragma unroll
                for (int m = 0; m < MAXB; ++m) {
                    for (int64_t j = st[m] + 1; j < en[m]; j += 4) {
                        uint4 v[4];
                        float w[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const bool ok = j + u < en[m];
                            const int64_t idx = a.indices[ok ? j + u : st[m]];
                            w[u] = (WEIGHTED && ok) ? a.weights[j + u] : 1.f;
                            v[u] = load_row_chunk(tab[m], idx, a.row_bytes);
                        }
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (j + u < en[m]) accumulate<DT, WEIGHTED>(acc[m], v[u], w[u]);
                    }
                }
#pragma unroll
                for (int m = 0; m < MAXB; ++m) {
                    if (en[m] >= 0) {
                        float *dst = X + (static_cast<size_t>(ss[m]) * N + tt[m] + 1) * XS + c * EPC;
#pragma unroll
                        for (int e = 0; e < EPC; e += 4)
                            *reinterpret_cast<float4 *>(dst + e) =
                                make_float4(acc[m][e], acc[m][e + 1], acc[m][e + 2], acc[m][e + 3]);
                    }
                }
            }
        }
    }
    __syncthreads();

    const int P = a.P, W = P + D;
    if constexpr (D == 64 || D == 128 || D == 256) {
        if constexpr (KSPLIT) {  // small N: the k-split Gram, one sample per wave
            if (gram_rows(N) == 9) lds_ksplit<9, D / 64>(a, X, XS, Sb, b0, wv, lane);
            else lds_ksplit<11, D / 64>(a, X, XS, Sb, b0, wv, lane);
            for (int i = tid; i < Sb * D; i += 256) {
                const int s = i / D, d = i - s * D;
                a.out[(static_cast<uint64_t>(b0) + s) * W + P + d] = X[static_cast<size_t>(s) * N * XS + d];
            }
            return;
        }
    }
    // ---- Gram blocks on the matrix cores; one upper 16 x 16 block per wave and job
    const int r16 = lane & 15, q = lane >> 4;
    for (int j = wv; j < Sb * a.NBLK; j += 4) {
        const int s = j / a.NBLK;
        int I, J;
        upper_block(j - s * a.NBLK, a.NB, I, J);
        const int ri = I * 16 + r16, rj = J * 16 + r16;
        const float *xs = X + static_cast<size_t>(s) * N * XS;
        const float *pi = xs + static_cast<size_t>(ri < N ? ri : 0) * XS + q * PL;
        const float *pj = xs + static_cast<size_t>(rj < N ? rj : 0) * XS + q * PL;
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            float xi[PL], xj[PL];
#pragma unroll
            for (int v = 0; v < PL; v += 4) {
                float4 f = ri < N ? *reinterpret_cast<const float4 *>(pi + ch * KC + v) : make_float4(0.f, 0.f, 0.f, 0.f);
                xi[v] = f.x, xi[v + 1] = f.y, xi[v + 2] = f.z, xi[v + 3] = f.w;
                f = rj < N ? *reinterpret_cast<const float4 *>(pj + ch * KC + v) : make_float4(0.f, 0.f, 0.f, 0.f);
                xj[v] = f.x, xj[v + 1] = f.y, xj[v + 2] = f.z, xj[v + 3] = f.w;
            }
#pragma unroll
            for (int e = 0; e < PL; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xi[e], xj[e], acc, 0, 0, 0);
        }
        // element (row 4q + v, column r16) of the block
        float *orow = a.out + (static_cast<uint64_t>(b0) + s) * W;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int gi = I * 16 + q * 4 + v, gj = J * 16 + r16;
            if (gi < gj && gj < N) orow[triu_pos(gi, gj, N)] = acc[v];
        }
    }
    // ---- the dense vector after the triangle
    for (int i = tid; i < Sb * D; i += 256) {
        const int s = i / D, d = i - s * D;
        a.out[(static_cast<uint64_t>(b0) + s) * W + P + d] = X[static_cast<size_t>(s) * N * XS + d];
    }
}

// Short bags (fewer than 4 lookups per bag on average), N <= 32: no LDS.  Each wavefront owns
// M samples and holds their X in registers in the matrix-core operand layout of the unfused
// interaction: lane (r16, q) pools rows I*16 + r16 of X itself, columns c*KC + q*KC/4 + e, and
// sums its bag's rows in order from zero as the unfused lane-group-per-bag pooling does.  The
// matrix-core sequence is then the unfused one, so the bits are the same.
//
// The M samples go through each dependent load step together (offsets, then first indices, then
// rows).  Every load of a step is unconditional -- addresses are selected, not branched on, and
// point at a valid location (row 0, sample B-1, the offsets array) where the value is unused --
// so the compiler issues them back to back and waits once per step.
__device__ __forceinline__ uint4 gload16(const void *p) {
    const u32x4 v = *(const DLRM_GLOBAL u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int DT, int NB, int KC, int NCH, int M, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_emb_interact_fwd_regs(FusedArgs a) {
    constexpr int D = KC * NCH;
    constexpr int PL = KC / 4;
    constexpr int NBLK = NB * (NB + 1) / 2;
    constexpr int ES = DT == DLRM_BF16 ? 2 : 4;
    constexpr int TW = PL * ES / 16;  // 16-byte loads per chunk of a table row quarter (1 or 2)
    constexpr int DW = PL / 4;        // 16-byte loads per chunk of a dense row quarter (2)
    const uint32_t b0 = (blockIdx.x * 4 + wave_id()) * M;
    if (b0 >= a.B) return;
    const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
    const int N = a.N;
    const int64_t *idx_base = a.indices ? a.indices : a.offsets;  // nnz = 0: never read for a value

    // step 1: bag bounds of every (sample, row block) of this lane
    int64_t j0[M][NB], j1[M][NB];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            const int i = R * 16 + r16;
            const uint32_t b = min(b0 + m, a.B - 1);
            const bool pooled_row = i >= 1 && i < N;
            const uint64_t bag = pooled_row ? static_cast<uint64_t>(i - 1) * a.B + b : 0;
            j0[m][R] = a.offsets[bag];
            j1[m][R] = a.offsets[bag + 1];
        }
    bool has[M][NB];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            const int i = R * 16 + r16;
            has[m][R] = i >= 1 && i < N && b0 + m < a.B && j0[m][R] < j1[m][R];
        }
    // step 2: first index (and weight) of each bag
    int64_t idx0[M][NB];
    float w0[M][NB];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            const int64_t jj = has[m][R] ? j0[m][R] : 0;
            idx0[m][R] = idx_base[jj];
            if constexpr (WEIGHTED) w0[m][R] = a.weights[has[m][R] ? jj : 0];
        }
    // step 3: the dense rows and the first row of every bag, all in flight together
    float x[M][NB][NCH][PL];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            const int i = R * 16 + r16;
            const uint32_t b = min(b0 + m, a.B - 1);
            const int t = i >= 1 && i < N ? i - 1 : 0;
            const char *trow = a.tables[t] + static_cast<uint64_t>(has[m][R] ? idx0[m][R] : 0) * a.row_bytes + q * PL * ES;
            const float *drow = a.dense + static_cast<uint64_t>(b) * D + q * PL;
            uint4 tv[NCH][TW], dv[NCH][DW];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
#pragma unroll
                for (int k = 0; k < TW; ++k) tv[c][k] = gload16(trow + (c * KC) * ES + 16 * k);
#pragma unroll
                for (int k = 0; k < DW; ++k) dv[c][k] = gload16(drow + c * KC + 4 * k);
            }
            const bool dense_row = i == 0;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                float tf[PL], df[PL];
#pragma unroll
                for (int k = 0; k < DW; ++k)
                    df[4 * k] = __uint_as_float(dv[c][k].x), df[4 * k + 1] = __uint_as_float(dv[c][k].y),
                    df[4 * k + 2] = __uint_as_float(dv[c][k].z), df[4 * k + 3] = __uint_as_float(dv[c][k].w);
                if constexpr (DT == DLRM_BF16) {
                    const uint32_t h[4] = {tv[c][0].x, tv[c][0].y, tv[c][0].z, tv[c][0].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) tf[2 * k] = bf16_lo(h[k]), tf[2 * k + 1] = bf16_hi(h[k]);
                } else {
#pragma unroll
                    for (int k = 0; k < TW; ++k)
                        tf[4 * k] = __uint_as_float(tv[c][k].x), tf[4 * k + 1] = __uint_as_float(tv[c][k].y),
                        tf[4 * k + 2] = __uint_as_float(tv[c][k].z), tf[4 * k + 3] = __uint_as_float(tv[c][k].w);
                }
#pragma unroll
                for (int e = 0; e < PL; ++e) {
                    const float p = WEIGHTED ? fmaf(w0[m][R], tf[e], 0.f) : 0.f + tf[e];
                    x[m][R][c][e] = dense_row ? df[e] : (has[m][R] ? p : 0.f);
                }
            }
        }
    // step 4: the remaining rows of bags with more than one lookup, in order
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            if (has[m][R] && j1[m][R] - j0[m][R] > 1) {
                const int i = R * 16 + r16;
                const char *tab = a.tables[i - 1] + q * PL * ES;
                for (int64_t j = j0[m][R] + 1; j < j1[m][R]; ++j) {
                    const char *row = tab + static_cast<uint64_t>(a.indices[j]) * a.row_bytes;
                    const float w = WEIGHTED ? a.weights[j] : 1.f;
#pragma unroll
                    for (int c = 0; c < NCH; ++c) {
                        float v[PL];
                        if constexpr (DT == DLRM_BF16) {
                            const uint4 u = gload16(row + (c * KC) * ES);
                            const uint32_t h[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                            for (int k = 0; k < 4; ++k) v[2 * k] = bf16_lo(h[k]), v[2 * k + 1] = bf16_hi(h[k]);
                        } else {
#pragma unroll
                            for (int k = 0; k < TW; ++k) {
                                const uint4 u = gload16(row + (c * KC) * ES + 16 * k);
                                v[4 * k] = __uint_as_float(u.x), v[4 * k + 1] = __uint_as_float(u.y),
                                v[4 * k + 2] = __uint_as_float(u.z), v[4 * k + 3] = __uint_as_float(u.w);
                            }
                        }
#pragma unroll
                        for (int e = 0; e < PL; ++e)
                            x[m][R][c][e] = WEIGHTED ? fmaf(w, v[e], x[m][R][c][e]) : x[m][R][c][e] + v[e];
                    }
                }
            }
        }
    // step 5: Gram blocks on the matrix cores, then [triu | dense]
    const int P = a.P;
    constexpr int ND = (D + kWave - 1) / kWave;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t b = b0 + m;
        if (b >= a.B) break;  // wave-uniform
        floatx4 acc[NBLK];
#pragma unroll
        for (int k = 0; k < NBLK; ++k) acc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < PL; ++e) {
                int k = 0;
#pragma unroll
                for (int I = 0; I < NB; ++I)
#pragma unroll
                    for (int J = I; J < NB; ++J, ++k)
                        acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[m][I][c][e], x[m][J][c][e], acc[k], 0, 0, 0);
            }
        float *orow = a.out + static_cast<uint64_t>(b) * (P + D);
        const float *dsrc = a.dense + static_cast<uint64_t>(b) * D;
        float dd[ND];
#pragma unroll
        for (int k = 0; k < ND; ++k) dd[k] = *(const DLRM_GLOBAL float *)(dsrc + min(lane + k * kWave, D - 1));
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
        for (int k2 = 0; k2 < ND; ++k2)
            if (lane + k2 * kWave < D) orow[P + lane + k2 * kWave] = dd[k2];
    }
}

__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), l);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32), l);
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Short bags, small N (N <= 11, D = 64 * CPL): pooled straight into the k-split Gram of gram.h.
// Lane l owns columns l*CPL.. of every row of X; lane t < T reads the bounds and first index of
// bag (t, b), which the wave then takes as uniform values, so each row is one coalesced load
// whose base is uniform.  The bag's rows are summed in order from zero, as the unfused
// lane-group-per-bag pooling sums them, and the Gram is the unfused interaction's: the bits
// match the two-call path.  M samples per wave go through each dependent load step together.
template <int DT, int NR, int CPL, int M, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_emb_interact_fwd_ksplit(FusedArgs a) {
    constexpr int D = 64 * CPL;
    constexpr int ES = DT == DLRM_BF16 ? 2 : 4;
    constexpr int TMAX = NR - 1;
    const uint32_t b0 = (blockIdx.x * 4 + wave_id()) * M;
    if (b0 >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int T = a.T, N = a.N;
    const int64_t *idx_base = a.indices ? a.indices : a.offsets;  // nnz = 0: never read for a value

    // step 1: lane t < T reads the bounds of bag (t, b) for each sample
    int64_t j0[M], j1[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t b = min(b0 + m, a.B - 1);
        const int t = lane < T ? lane : T - 1;
        const uint64_t bag = static_cast<uint64_t>(t) * a.B + b;
        j0[m] = a.offsets[bag];
        j1[m] = a.offsets[bag + 1];
    }
    // step 2: first index and weight of that bag
    int64_t idx0[M];
    float w0[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const bool has = j0[m] < j1[m];
        idx0[m] = idx_base[has ? j0[m] : 0];
        if constexpr (WEIGHTED) w0[m] = a.weights[has ? j0[m] : 0];
        if (!has) idx0[m] = 0;
    }
    // step 3: dense rows and the first row of every bag, all in flight together
    float x[M][NR][CPL];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t b = min(b0 + m, a.B - 1);
        uint32_t dw[CPL];
        gload_words<CPL>(a.dense + static_cast<uint64_t>(b) * D + lane * CPL, dw);
#pragma unroll
        for (int c = 0; c < CPL; ++c) x[m][0][c] = __uint_as_float(dw[c]);
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            const int tt = t < T ? t : T - 1;
            const int64_t idx = readlane64(idx0[m], tt);
            const char *row = a.tables[tt] + static_cast<uint64_t>(idx) * a.row_bytes + lane * CPL * ES;
            float v[CPL];
            if constexpr (DT == DLRM_BF16) {
                if constexpr (CPL == 1) {
                    v[0] = __uint_as_float(static_cast<uint32_t>(*(const DLRM_GLOBAL uint16_t *)row) << 16);
                } else {
                    uint32_t h[CPL / 2];
                    gload_words<CPL / 2>(row, h);
#pragma unroll
                    for (int k = 0; k < CPL / 2; ++k) v[2 * k] = bf16_lo(h[k]), v[2 * k + 1] = bf16_hi(h[k]);
                }
            } else {
                uint32_t h[CPL];
                gload_words<CPL>(row, h);
#pragma unroll
                for (int c = 0; c < CPL; ++c) v[c] = __uint_as_float(h[c]);
            }
            const bool has = t < T && readlane64(j0[m], tt) < readlane64(j1[m], tt);
            const float w = WEIGHTED ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0[m]), tt)) : 1.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const float p = WEIGHTED ? fmaf(w, v[c], 0.f) : 0.f + v[c];
                x[m][t + 1][c] = has ? p : 0.f;
            }
        }
    }
    // step 4: the remaining rows of bags with more than one lookup, in order (uniform loops)
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t >= T || b0 + m >= a.B) continue;
            const int64_t s0 = readlane64(j0[m], t), s1 = readlane64(j1[m], t);
            const char *tab = a.tables[t] + lane * CPL * ES;
            for (int64_t j = s0 + 1; j < s1; ++j) {
                const char *row = tab + static_cast<uint64_t>(a.indices[j]) * a.row_bytes;
                const float w = WEIGHTED ? a.weights[j] : 1.f;
                float v[CPL];
                if constexpr (DT == DLRM_BF16) {
                    if constexpr (CPL == 1) {
                        v[0] = __uint_as_float(static_cast<uint32_t>(*(const DLRM_GLOBAL uint16_t *)row) << 16);
                    } else {
                        uint32_t h[CPL / 2];
                        gload_words<CPL / 2>(row, h);
#pragma unroll
                        for (int k = 0; k < CPL / 2; ++k) v[2 * k] = bf16_lo(h[k]), v[2 * k + 1] = bf16_hi(h[k]);
                    }
                } else {
                    uint32_t h[CPL];
                    gload_words<CPL>(row, h);
#pragma unroll
                    for (int c = 0; c < CPL; ++c) v[c] = __uint_as_float(h[c]);
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    x[m][t + 1][c] = WEIGHTED ? fmaf(w, v[c], x[m][t + 1][c]) : x[m][t + 1][c] + v[c];
            }
        }
    // step 5: the Gram and [triu | dense]
    int pi, pj;
    const bool holds = gram_lane_pair<NR>(lane, pi, pj);
    const int P = a.P;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t b = b0 + m;
        if (b >= a.B) break;  // wave-uniform
        const float z = gram_ksplit<NR, CPL>(x[m]);
        float *orow = a.out + static_cast<uint64_t>(b) * (P + D);
        if (holds && pj < N) orow[triu_pos(pi, pj, N)] = z;
#pragma unroll
        for (int c = 0; c < CPL; ++c) orow[P + lane * CPL + c] = x[m][0][c];
    }
}

template <int DT>
void dispatch_ksplit(const FusedArgs &a, int D, bool weighted, hipStream_t stream) {
#define DLRM_KSPLIT(NR, CPL, M)                                                                                     \
    do {                                                                                                            \
        const dim3 grid(static_cast<uint32_t>((a.B + 4 * (M) - 1) / (4 * (M)))), block(256);                       \
        if (weighted) DLRM_LAUNCH("emb_interact_fwd_ksplit", (k_emb_interact_fwd_ksplit<DT, NR, CPL, M, true>), grid, block, 0, stream, a); \
        else DLRM_LAUNCH("emb_interact_fwd_ksplit", (k_emb_interact_fwd_ksplit<DT, NR, CPL, M, false>), grid, block, 0, stream, a); \
    } while (0)
    if (gram_rows(a.N) == 9) {
        if (D == 64) DLRM_KSPLIT(9, 1, DLRM_FUSED_M);
        else if (D == 128) DLRM_KSPLIT(9, 2, DLRM_FUSED_M);
        else DLRM_KSPLIT(9, 4, 1);
    } else {
        if (D == 64) DLRM_KSPLIT(11, 1, DLRM_FUSED_M);
        else if (D == 128) DLRM_KSPLIT(11, 2, DLRM_FUSED_M);
        else DLRM_KSPLIT(11, 4, 1);
    }
#undef DLRM_KSPLIT
}

// The register path for D = KC * NCH and NB row blocks (NB * D <= 256); M samples per wave.
template <int DT, int NB>
bool dispatch_regs(const FusedArgs &a, int D, bool weighted, hipStream_t stream) {
#define DLRM_REGS(KC, NCH)                                                                                          \
    do {                                                                                                            \
        constexpr int M_ = NB * KC * NCH <= 128 ? DLRM_FUSED_M : 1;                                                 \
        const dim3 grid(static_cast<uint32_t>((a.B + 4 * M_ - 1) / (4 * M_))), block(256);                          \
        if (weighted) DLRM_LAUNCH("emb_interact_fwd_regs", (k_emb_interact_fwd_regs<DT, NB, KC, NCH, M_, true>), grid, block, 0, stream, a); \
        else DLRM_LAUNCH("emb_interact_fwd_regs", (k_emb_interact_fwd_regs<DT, NB, KC, NCH, M_, false>), grid, block, 0, stream, a); \
    } while (0)
    switch (D) {
        case 16: if constexpr (DT == DLRM_F32) { DLRM_REGS(16, 1); return true; } return false;
        case 32: DLRM_REGS(32, 1); return true;
        case 64: DLRM_REGS(32, 2); return true;
        case 128: DLRM_REGS(32, 4); return true;
        case 256: if constexpr (NB == 1) { DLRM_REGS(32, 8); return true; } return false;
        default: return false;
    }
#undef DLRM_REGS
}

template <int DT, int G, int KC, bool W, bool WPB>
void launch_fused(const FusedArgs &a, size_t lds, uint32_t blocks, hipStream_t stream) {
    constexpr int D = G * Elem<DT>::kPerChunk;
    if constexpr (D == 64 || D == 128 || D == 256) {
        if (a.ksplit) {
            DLRM_LAUNCH("emb_interact_fwd", (k_emb_interact_fwd<DT, G, KC, W, WPB, true>), dim3(blocks), dim3(256), lds, stream, a);
            return;
        }
    }
    DLRM_LAUNCH("emb_interact_fwd", (k_emb_interact_fwd<DT, G, KC, W, WPB, false>), dim3(blocks), dim3(256), lds, stream, a);
}

template <int DT, int G, int KC>
void dispatch_mode(const FusedArgs &a, size_t lds, uint32_t blocks, bool weighted, bool wpb,
                   hipStream_t stream) {
    if (wpb) {
        if (weighted) launch_fused<DT, G, KC, true, true>(a, lds, blocks, stream);
        else launch_fused<DT, G, KC, false, true>(a, lds, blocks, stream);
    } else {
        if (weighted) launch_fused<DT, G, KC, true, false>(a, lds, blocks, stream);
        else launch_fused<DT, G, KC, false, false>(a, lds, blocks, stream);
    }
}

// G = 16-byte chunks per row; KC as the unfused interaction chooses it (16 for D = 16, else 32).
template <int DT>
bool dispatch_fused(const FusedArgs &a, size_t lds, uint32_t blocks, bool weighted, bool wpb,
                    hipStream_t stream) {
    constexpr int EPC = Elem<DT>::kPerChunk;
    switch (a.row_bytes / 16) {
        case 4:
            if constexpr (4 * EPC == 16) dispatch_mode<DT, 4, 16>(a, lds, blocks, weighted, wpb, stream);
            else dispatch_mode<DT, 4, 32>(a, lds, blocks, weighted, wpb, stream);
            return true;
        case 8: dispatch_mode<DT, 8, 32>(a, lds, blocks, weighted, wpb, stream); return true;
        case 16: dispatch_mode<DT, 16, 32>(a, lds, blocks, weighted, wpb, stream); return true;
        case 32: dispatch_mode<DT, 32, 32>(a, lds, blocks, weighted, wpb, stream); return true;
        case 64: dispatch_mode<DT, 64, 32>(a, lds, blocks, weighted, wpb, stream); return true;
        default: return false;
    }
}

constexpr size_t kMaxFusedLds = 64 * 1024;

}  // namespace
}  // namespace dlrm

extern "C" int emb_bag_interact_fwd(const void *const *tables, const int64_t *rows, int32_t T,
                                    int32_t D, int32_t dtype, const int64_t *indices,
                                    const int64_t *offsets, const float *per_sample_weights,
                                    int64_t B, int64_t nnz, const float *dense, float *out,
                                    uint32_t flags, dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc = check_batch(tables, rows, T, D, dtype, indices, offsets, DLRM_INDEX_I64, per_sample_weights, B, nnz);
    if (rc != DLRM_OK) return rc;
    if (flags & ~DLRM_FLAG_CHECK_INDICES) return DLRM_ERR_INVALID_ARG;
    const int N = T + 1;
    const uint32_t row_bytes = static_cast<uint32_t>(D * elem_size(dtype));
    const uint32_t chunks = row_bytes / 16;
    if (D % 16 != 0 || (chunks & (chunks - 1)) != 0 || chunks < 4 || chunks > 64) return DLRM_ERR_UNSUPPORTED;
    if (fused_lds_bytes(1, N, D, T) > kMaxFusedLds) return DLRM_ERR_UNSUPPORTED;
    if (B >= (int64_t(1) << 31) / 4) return DLRM_ERR_UNSUPPORTED;
    if (B == 0) return nnz == 0 ? DLRM_OK : DLRM_ERR_INVALID_ARG;
    if (!dense || !out || !aligned(dense, 16) || !aligned(out, 4)) return DLRM_ERR_INVALID_ARG;
    if (flags & DLRM_FLAG_CHECK_INDICES) {
        // the output buffer lends 4 bytes for the flag; it is overwritten below
        rc = check_csr_on_device(rows, T, indices, offsets, DLRM_INDEX_I64, B, nnz, reinterpret_cast<int *>(out), stream);
        if (rc != DLRM_OK) return rc;
    }
    FusedArgs a{};
    for (int t = 0; t < T; ++t) a.tables[t] = static_cast<const char *>(tables[t]);
    a.indices = indices;
    a.offsets = offsets;
    a.weights = per_sample_weights;
    a.dense = dense;
    a.out = out;
    a.B = static_cast<uint32_t>(B);
    a.T = T;
    a.N = N;
    a.P = N * (N - 1) / 2;
    a.NB = (N + 15) / 16;
    a.NBLK = a.NB * (a.NB + 1) / 2;
    a.row_bytes = row_bytes;
    // the same kernel choice as emb_bag_fwd: a wavefront per bag for 4+ lookups per bag on average
    const bool wpb = nnz >= 4 * static_cast<int64_t>(T) * B;
    const bool weighted = per_sample_weights != nullptr && nnz > 0;  // no lookup: nothing to weigh
    a.ksplit = gram_ksplit_ok(N, D) ? 1 : 0;
    if (!wpb && a.ksplit) {  // short bags, small N: pooled straight into the k-split Gram
        if (dtype == DLRM_F32) dispatch_ksplit<DLRM_F32>(a, D, weighted, stream);
        else dispatch_ksplit<DLRM_BF16>(a, D, weighted, stream);
        return launch_status();
    }
    if (!wpb && a.NB <= 2 && a.NB * D <= 256) {  // short bags, X fits in registers: no LDS, no barriers
        const bool ok = dtype == DLRM_F32
                            ? (a.NB == 1 ? dispatch_regs<DLRM_F32, 1>(a, D, weighted, stream)
                                         : dispatch_regs<DLRM_F32, 2>(a, D, weighted, stream))
                            : (a.NB == 1 ? dispatch_regs<DLRM_BF16, 1>(a, D, weighted, stream)
                                         : dispatch_regs<DLRM_BF16, 2>(a, D, weighted, stream));
        if (ok) return launch_status();
    }
    const int NG = kWave / static_cast<int>(chunks);
    int S = 1;
    if (!wpb) {  // lane group per bag: enough bags per block for all 4*NG groups, at most 4 samples
        S = (4 * NG + T - 1) / T;
        S = S < 1 ? 1 : (S > 4 ? 4 : S);
        while (S > 1 && fused_lds_bytes(S, N, D, T) > kMaxFusedLds) --S;
    }
    a.S = S;
    a.BPG = (S * T + 4 * NG - 1) / (4 * NG);
    const size_t lds = fused_lds_bytes(S, N, D, T);
    const uint32_t blocks = static_cast<uint32_t>((B + S - 1) / S);
    const bool ok = dtype == DLRM_F32 ? dispatch_fused<DLRM_F32>(a, lds, blocks, weighted, wpb, stream)
                                      : dispatch_fused<DLRM_BF16>(a, lds, blocks, weighted, wpb, stream);
    if (!ok) return DLRM_ERR_UNSUPPORTED;
    return launch_status();
}
