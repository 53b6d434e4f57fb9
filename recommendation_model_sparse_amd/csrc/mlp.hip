// Dense layers either side of the sparse path (robocikowo.com "DLRM", paragraph "Forward pass":
// stage (1) bottom MLP, stage (4) top MLP with the sigmoid, trained on cross-entropy with
// SGD/Adagrad).
//
// The GEMMs are plain library GEMMs and run in hipBLASLt (bf16 operands, fp32 accumulation,
// bias + ReLU fused into its epilogue on the forward).  The rest is hand-written here:
//   - ReLU backward + bf16 rounding of dz for the GEMMs + per-block partial column sums of the
//     fp32 dz, then a fixed-order reduction to the bias gradient (deterministic, no atomics);
//   - the one-unit sigmoid head with the mean binary cross-entropy, forward and backward in one
//     pass: a wavefront per row, the dot product reduced across the wave, per-block partial sums of
//     dw, db and the loss reduced in a fixed order;
//   - SGD on fp32 master weights refreshing their bf16 copies, and a row cast / pad.
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "common.h"
#include "dlrm_mlp.h"

namespace dlrm {
namespace {

constexpr size_t kGemmScratch = size_t(32) << 20;  // hipBLASLt workspace per GEMM
constexpr int kGradRows = 32;                       // rows per block of the bias-gradient partials
constexpr int kHeadBlocks = 512;                    // blocks of the head (fixes its summation order)
constexpr int kHeadMaxK = 1024;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));  // nearest even
}

// ---------------------------------------------------------------- ReLU backward + bias gradient

// Block (bx, by): rows [bx*kGradRows, +kGradRows), columns 4*(by*256 + g) .. +3 for the block's
// column groups g (N % 8 == 0, so a group's 4 columns are 16 bytes of dy, 8 bytes of a bf16 y and
// of dz: vector accesses, a quarter of the instructions of one column per thread).  A layer
// narrower than 1024 columns has fewer than 256 groups: the block's threads then split its rows
// into RL = 256 / groups interleaved row lanes (lane j takes rows r0 + j, r0 + j + RL, ...), so
// every thread has work and the block's rows are walked RL at a time.  dz = dy * [y > 0] (or dy);
// dz rounded to bf16; partial[bx][c] = sum of the block's fp32 dz of column c: each row lane adds
// its rows in order, then the lanes' sums are added in lane order.
template <bool RELU, int YT>
__global__ __launch_bounds__(256) void k_relu_grad(const float *__restrict__ dy, const void *__restrict__ y,
                                                   int64_t M, int32_t N, uint16_t *__restrict__ dz,
                                                   float *__restrict__ partial) {
    __shared__ float4 lane_sum[256];
    const int32_t groups = min(N / 4, 256);  // column groups per block
    const int RL = 256 / groups;             // row lanes
    const int tid = threadIdx.x, j = tid / groups, g = tid % groups;
    const int32_t c = (blockIdx.y * 256 + g) * 4;
    const bool active = j < RL && c < N;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kGradRows;
    const int64_t r1 = min<int64_t>(r0 + kGradRows, M);
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    constexpr int R = 8;  // rows whose loads are in flight together (unconditional: clamped rows)
    // a lane's rows r0 + j + RL*k; the last one it has is clamped to in every batch
    const int64_t rl = active && r0 + j < r1 ? r1 - 1 - (r1 - 1 - r0 - j) % RL : -1;
    for (int64_t r = r0 + j; active && r < r1; r += static_cast<int64_t>(R) * RL) {
        float4 g4[R];
        float yv[R][4];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const uint64_t i = static_cast<uint64_t>(min(r + static_cast<int64_t>(u) * RL, rl)) * N + c;
            g4[u] = *reinterpret_cast<const float4 *>(dy + i);
            if constexpr (RELU) {
                if constexpr (YT == DLRM_F32) {
                    const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(y) + i);
                    yv[u][0] = f.x, yv[u][1] = f.y, yv[u][2] = f.z, yv[u][3] = f.w;
                } else {
                    const uint2 h = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(y) + i);
                    yv[u][0] = __uint_as_float(h.x << 16), yv[u][1] = __uint_as_float(h.x & 0xffff0000u);
                    yv[u][2] = __uint_as_float(h.y << 16), yv[u][3] = __uint_as_float(h.y & 0xffff0000u);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int64_t ru = r + static_cast<int64_t>(u) * RL;
            if (ru >= r1) break;
            float gu[4] = {g4[u].x, g4[u].y, g4[u].z, g4[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (RELU) gu[e] = yv[u][e] > 0.f ? gu[e] : 0.f;
                s[e] += gu[e];
            }
            const uint2 o = make_uint2(static_cast<uint32_t>(f32_to_bf16(gu[0])) | (static_cast<uint32_t>(f32_to_bf16(gu[1])) << 16),
                                       static_cast<uint32_t>(f32_to_bf16(gu[2])) | (static_cast<uint32_t>(f32_to_bf16(gu[3])) << 16));
            *reinterpret_cast<uint2 *>(dz + static_cast<uint64_t>(ru) * N + c) = o;
        }
    }
    if (RL == 1) {  // block-uniform: one lane per column group, no combine
        if (active)
            *reinterpret_cast<float4 *>(partial + static_cast<uint64_t>(blockIdx.x) * N + c) =
                make_float4(s[0], s[1], s[2], s[3]);
        return;
    }
    lane_sum[tid] = make_float4(s[0], s[1], s[2], s[3]);
    __syncthreads();
    if (j == 0 && c < N) {
        float4 t = lane_sum[g];
        for (int q = 1; q < RL; ++q) {
            const float4 v = lane_sum[q * groups + g];
            t.x += v.x, t.y += v.y, t.z += v.z, t.w += v.w;
        }
        *reinterpret_cast<float4 *>(partial + static_cast<uint64_t>(blockIdx.x) * N + c) = t;
    }
}

// Sum over blocks of partial[blk][c] (row stride `ld`) for column c: one wavefront per column;
// lane l adds blocks l, l+64, ... in order, then a fixed butterfly adds the 64 lane sums.  A lane's
// blocks are loaded LB at a time (clamped in bounds) before they are added, so LB of them make one
// round trip together; the order of the additions is the same.
__device__ __forceinline__ float wave_colsum(const float *__restrict__ partial, int32_t nblk, int64_t ld,
                                             int64_t c) {
    constexpr int LB = 8;
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    for (int32_t k0 = lane; k0 < nblk; k0 += LB * kWave) {
        float v[LB];
#pragma unroll
        for (int u = 0; u < LB; ++u) v[u] = partial[static_cast<uint64_t>(min(k0 + u * kWave, nblk - 1)) * ld + c];
#pragma unroll
        for (int u = 0; u < LB; ++u)
            if (k0 + u * kWave < nblk) s += v[u];
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) s += __shfl_xor(s, sh);
    return s;
}

// ---------------------------------------------------------------- sigmoid head + BCE

// Layout of the head's partials: [kHeadBlocks][K + 2] (dw columns, then db, then loss).
// Lane l holds the CPL consecutive columns l*CPL .. l*CPL+CPL-1 of a row (one vector access of
// 2*CPL bytes of x, 4*CPL of dx); CPL = K/64 rounded up to a power of two.  K % 8 == 0, so for
// CPL >= 8 each 8-column piece is either wholly inside the row or wholly past it, and for CPL <= 4
// a lane's columns are all inside iff its first one is.  Each wave takes kHeadRows rows at once
// (its grid-stride rows m, m + nw, ...), whose loads are in flight together.
constexpr int kHeadRows = 4;

template <int CPL>
__device__ __forceinline__ void head_load(const uint16_t *p, int lane, int32_t K, float *x) {
    const int c0 = lane * CPL;
    if constexpr (CPL >= 8) {
#pragma unroll
        for (int j = 0; j < CPL / 8; ++j) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c0 + 8 * j < K) v = *reinterpret_cast<const uint4 *>(p + c0 + 8 * j);
            const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * j + 2 * e] = __uint_as_float(q[e] << 16);
                x[8 * j + 2 * e + 1] = __uint_as_float(q[e] & 0xffff0000u);
            }
        }
    } else if constexpr (CPL == 4) {
        uint2 v = make_uint2(0, 0);
        if (c0 < K) v = *reinterpret_cast<const uint2 *>(p + c0);
        x[0] = __uint_as_float(v.x << 16), x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16), x[3] = __uint_as_float(v.y & 0xffff0000u);
    } else if constexpr (CPL == 2) {
        uint32_t v = 0;
        if (c0 < K) v = *reinterpret_cast<const uint32_t *>(p + c0);
        x[0] = __uint_as_float(v << 16), x[1] = __uint_as_float(v & 0xffff0000u);
    } else {
        x[0] = c0 < K ? bf16_to_f32(p[c0]) : 0.f;
    }
}

template <int CPL>
__global__ __launch_bounds__(256) void k_bce_head(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                  const float *__restrict__ b, const float *__restrict__ t,
                                                  int64_t M, int32_t K, float *__restrict__ p,
                                                  float *__restrict__ dx, float *__restrict__ partial) {
    __shared__ float red[4][kHeadMaxK + 2];
    const int lane = threadIdx.x & 63, wv = static_cast<int>(wave_id());
    const int c0 = lane * CPL;
    const float bias = b[0];
    const float invM = 1.0f / static_cast<float>(M);
    float wl[CPL], dwl[CPL];
    head_load<CPL>(w, lane, K, wl);
#pragma unroll
    for (int i = 0; i < CPL; ++i) dwl[i] = 0.f;
    float dbl = 0.f, lossl = 0.f;
    const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
    for (int64_t m0 = static_cast<int64_t>(blockIdx.x) * 4 + wv; m0 < M; m0 += nw * kHeadRows) {  // wave-uniform
        float xv[kHeadRows][CPL], z[kHeadRows], tm[kHeadRows];
#pragma unroll
        for (int r = 0; r < kHeadRows; ++r) {  // rows past M re-read the last row; their results are dropped
            const int64_t m = min(m0 + r * nw, M - 1);
            head_load<CPL>(x + static_cast<uint64_t>(m) * K, lane, K, xv[r]);
            tm[r] = t[m];
        }
#pragma unroll
        for (int r = 0; r < kHeadRows; ++r) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) s = fmaf(xv[r][i], wl[i], s);
            z[r] = s;
        }
#pragma unroll
        for (int sh = 32; sh >= 1; sh >>= 1)
#pragma unroll
            for (int r = 0; r < kHeadRows; ++r) z[r] += __shfl_xor(z[r], sh);  // every lane: the same bits
#pragma unroll
        for (int r = 0; r < kHeadRows; ++r) {
            const int64_t m = m0 + r * nw;
            if (m >= M) break;  // wave-uniform
            const float zr = z[r] + bias;
            const float pm = 1.0f / (1.0f + expf(-zr));
            const float loss = fmaxf(zr, 0.f) - zr * tm[r] + log1pf(expf(-fabsf(zr)));
            const float dz = (pm - tm[r]) * invM;
            if (lane == 0) p[m] = pm;
            float *dxr = dx + static_cast<uint64_t>(m) * K + c0;
            float o[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                o[i] = dz * wl[i];
                dwl[i] = fmaf(dz, xv[r][i], dwl[i]);
            }
            if constexpr (CPL >= 4) {
#pragma unroll
                for (int j = 0; j < CPL / 4; ++j)
                    if (c0 + 4 * j < K)
                        *reinterpret_cast<float4 *>(dxr + 4 * j) = make_float4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
            } else if constexpr (CPL == 2) {
                if (c0 < K) *reinterpret_cast<float2 *>(dxr) = make_float2(o[0], o[1]);
            } else {
                if (c0 < K) dxr[0] = o[0];
            }
            dbl += dz;
            lossl += loss;
        }
    }
    // combine the block's 4 waves in order, then write the block's partials
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        if (c0 + i < K) red[wv][c0 + i] = dwl[i];
    if (lane == 0) {
        red[wv][K] = dbl;
        red[wv][K + 1] = lossl;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < K + 2; c += 256) {
        const float s = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
        partial[static_cast<uint64_t>(blockIdx.x) * (K + 2) + c] = s;
    }
}

__global__ __launch_bounds__(256) void k_bce_final(const float *__restrict__ partial, int32_t nblk, int32_t K,
                                                   int64_t M, float *__restrict__ dw, float *__restrict__ db,
                                                   float *__restrict__ loss) {
    const int32_t c = blockIdx.x * 4 + static_cast<int32_t>(wave_id());
    if (c >= K + 2) return;  // wave-uniform
    const float s = wave_colsum(partial, nblk, K + 2, c);
    if ((threadIdx.x & 63) != 0) return;
    if (c < K) dw[c] = s;
    else if (c == K) db[0] = s;
    else loss[0] = s / static_cast<float>(M);
}

// ---------------------------------------------------------------- SGD and row casts

__global__ __launch_bounds__(256) void k_sgd_dense(float *__restrict__ w32, uint16_t *__restrict__ w16,
                                                   const float *__restrict__ g, int64_t n, float lr) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const float v = fmaf(-lr, g[i], w32[i]);
    w32[i] = v;
    if (w16) w16[i] = f32_to_bf16(v);
}

// Many SGD updates in one launch: tensor i owns blocks [boff[i], boff[i+1]), each block 1024
// consecutive elements (4 per thread, 256 apart), the same arithmetic as k_sgd_dense.
constexpr int kSgdMaxTensors = 64;
constexpr int kSgdPerBlock = 1024;
struct SgdMulti {
    float *w32[kSgdMaxTensors];
    uint16_t *w16[kSgdMaxTensors];
    const float *g[kSgdMaxTensors];
    int64_t n[kSgdMaxTensors];
    uint32_t boff[kSgdMaxTensors + 1];
    int32_t count;
    float lr;
};

__global__ __launch_bounds__(256) void k_sgd_dense_multi(SgdMulti a) {
    int i = 0;  // the tensor of this block (uniform scan over at most 64 entries)
    while (i + 1 < a.count && blockIdx.x >= a.boff[i + 1]) ++i;
    const int64_t base = static_cast<int64_t>(blockIdx.x - a.boff[i]) * kSgdPerBlock + threadIdx.x;
    float *w32 = a.w32[i];
    uint16_t *w16 = a.w16[i];
    const float *g = a.g[i];
#pragma unroll
    for (int k = 0; k < kSgdPerBlock / 256; ++k) {
        const int64_t e = base + k * 256;
        if (e < a.n[i]) {
            const float v = fmaf(-a.lr, g[e], w32[e]);
            w32[e] = v;
            if (w16) w16[e] = f32_to_bf16(v);
        }
    }
}

// Block (bx, by) casts columns [by*1024, by*1024 + 1024) of its rows; its 256 threads are G column
// groups (G = 256, or a narrower row's (dst_cols + 3) / 4) times RL = 256 / G row lanes, and lane j
// takes the rows bx*RL*NR + j + RL*u, u < NR, all NR rows' loads in flight together (NR = 8, fewer
// for narrow rows so the launch keeps enough blocks).  Columns from `cols` to dst_cols are zero.
// VEC (dst_cols % 4 == 0, 16-byte aligned dst): group g holds 4 consecutive columns, stored as one
// vector; otherwise group g holds columns g, g + G, g + 2G, g + 3G, so each scalar access of the
// wavefront is contiguous.
constexpr int kCastRowsPerLane = 8;

inline int32_t cast_groups(int32_t dst_cols) { return std::min((dst_cols + 3) / 4, 256); }
inline int cast_rows_per_lane(int32_t dst_cols) {
    const int RL = 256 / cast_groups(dst_cols);
    return RL >= 64 ? 1 : std::min(kCastRowsPerLane, 64 / RL);
}

template <int ST, int DT, bool VEC>
__global__ __launch_bounds__(256) void k_cast_rows(const void *__restrict__ src, int64_t src_ld, int64_t M,
                                                   int32_t cols, void *__restrict__ dst, int32_t dst_cols,
                                                   int32_t rows_per_lane) {
    constexpr int R = kCastRowsPerLane;
    const int32_t G = min((dst_cols + 3) / 4, 256);
    const int RL = 256 / G;
    const int tid = threadIdx.x, j = tid / G, g = tid % G;
    if (j >= RL) return;  // no barrier follows
    const int32_t t0 = static_cast<int32_t>(blockIdx.y) * 1024;
    int32_t col[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) col[e] = t0 + (VEC ? 4 * g + e : g + e * G);
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * RL * rows_per_lane + j;
    float v[R][4];
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int64_t m = r0 + static_cast<int64_t>(u) * RL;
        const bool row = u < rows_per_lane && m < M;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[u][e] = 0.f;
            if (row && col[e] < cols) {
                const uint64_t s = static_cast<uint64_t>(m) * src_ld + col[e];
                v[u][e] = ST == DLRM_F32 ? static_cast<const float *>(src)[s]
                                         : bf16_to_f32(static_cast<const uint16_t *>(src)[s]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int64_t m = r0 + static_cast<int64_t>(u) * RL;
        if (u >= rows_per_lane || m >= M) break;
        const uint64_t d = static_cast<uint64_t>(m) * dst_cols;
        if constexpr (VEC) {
            if (col[0] < dst_cols) {
                if constexpr (DT == DLRM_F32) {
                    *reinterpret_cast<float4 *>(static_cast<float *>(dst) + d + col[0]) =
                        make_float4(v[u][0], v[u][1], v[u][2], v[u][3]);
                } else {
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(dst) + d + col[0]) = make_uint2(
                        static_cast<uint32_t>(f32_to_bf16(v[u][0])) | (static_cast<uint32_t>(f32_to_bf16(v[u][1])) << 16),
                        static_cast<uint32_t>(f32_to_bf16(v[u][2])) | (static_cast<uint32_t>(f32_to_bf16(v[u][3])) << 16));
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (col[e] >= dst_cols) continue;
                if constexpr (DT == DLRM_F32) static_cast<float *>(dst)[d + col[e]] = v[u][e];
                else static_cast<uint16_t *>(dst)[d + col[e]] = f32_to_bf16(v[u][e]);
            }
        }
    }
}


// ---------------------------------------------------------------- hipBLASLt

std::mutex g_lt_mutex;
hipblasLtHandle_t g_lt_handle[64] = {};

using AlgoKey = std::tuple<int, int, int, int64_t, int64_t, int64_t, int, int>;
std::map<AlgoKey, hipblasLtMatmulAlgo_t> g_algo_cache;

hipblasLtHandle_t lt_handle(int dev) {
    std::lock_guard<std::mutex> lock(g_lt_mutex);
    if (!g_lt_handle[dev] && hipblasLtCreate(&g_lt_handle[dev]) != HIPBLAS_STATUS_SUCCESS) g_lt_handle[dev] = nullptr;
    return g_lt_handle[dev];
}

// Column-major D[m][n] (ld m) = op(A) op(B) (+ bias[m], ReLU); A, B bf16, fp32 accumulation.
// With batch > 1: `batch` such products, operand s at A + s*sA, B + s*sB, D + s*sD (elements).
int lt_gemm(hipStream_t stream, bool transA, bool transB, int64_t m, int64_t n, int64_t k, const void *A,
            int64_t lda, const void *B, int64_t ldb, void *D, hipDataType dtype, const float *bias, bool relu,
            void *ws, size_t ws_bytes, int32_t batch = 1, int64_t sA = 0, int64_t sB = 0, int64_t sD = 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DLRM_ERR_HIP;
    hipblasLtHandle_t h = lt_handle(dev);
    if (!h) return DLRM_ERR_HIP;
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    int rc = DLRM_ERR_HIP;
    const hipblasOperation_t opA = transA ? HIPBLAS_OP_T : HIPBLAS_OP_N, opB = transB ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    const hipblasLtEpilogue_t epi = bias ? (relu ? HIPBLASLT_EPILOGUE_RELU_BIAS : HIPBLASLT_EPILOGUE_BIAS)
                                         : (relu ? HIPBLASLT_EPILOGUE_RELU : HIPBLASLT_EPILOGUE_DEFAULT);
    const hipDataType bias_type = HIP_R_32F;
    const float alpha = 1.f, beta = 0.f;
    do {
        if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opA, sizeof(opA)) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opB, sizeof(opB)) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) != HIPBLAS_STATUS_SUCCESS) break;
        if (bias) {
            if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) != HIPBLAS_STATUS_SUCCESS) break;
            if (hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type, sizeof(bias_type)) != HIPBLAS_STATUS_SUCCESS) break;
        }
        if (hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, transA ? k : m, transA ? m : k, lda) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, transB ? n : k, transB ? k : n, ldb) != HIPBLAS_STATUS_SUCCESS) break;
        if (hipblasLtMatrixLayoutCreate(&ld, dtype, m, n, m) != HIPBLAS_STATUS_SUCCESS) break;
        if (batch > 1) {
            bool ok = true;
            const hipblasLtMatrixLayout_t lays[3] = {la, lb, ld};
            const int64_t strides[3] = {sA, sB, sD};
            for (int q = 0; q < 3 && ok; ++q)
                ok = hipblasLtMatrixLayoutSetAttribute(lays[q], HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &batch,
                                                       sizeof(batch)) == HIPBLAS_STATUS_SUCCESS &&
                     hipblasLtMatrixLayoutSetAttribute(lays[q], HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET,
                                                       &strides[q], sizeof(strides[q])) == HIPBLAS_STATUS_SUCCESS;
            if (!ok) break;
        }
        const AlgoKey key{dev, (transA ? 1 : 0) | (transB ? 2 : 0), static_cast<int>(epi), m, n, k, static_cast<int>(dtype), batch};
        hipblasLtMatmulAlgo_t algo;
        bool have = false;
        {
            std::lock_guard<std::mutex> lock(g_lt_mutex);
            auto it = g_algo_cache.find(key);
            if (it != g_algo_cache.end()) algo = it->second, have = true;
        }
        if (!have) {
            if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) break;
            const uint64_t max_ws = ws_bytes;
            if (hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws,
                                                      sizeof(max_ws)) != HIPBLAS_STATUS_SUCCESS) break;
            constexpr int kCand = 8;
            hipblasLtMatmulHeuristicResult_t res[kCand];
            int found = 0;
            if (hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, ld, ld, pref, kCand, res, &found) !=
                    HIPBLAS_STATUS_SUCCESS ||
                found < 1) {
                rc = DLRM_ERR_UNSUPPORTED;
                break;
            }
            // first call for this shape: time every candidate on the caller's stream, keep the fastest
            int best = 0;
            if (found > 1) {
                hipEvent_t e0, e1;
                if (hipEventCreate(&e0) != hipSuccess) break;
                if (hipEventCreate(&e1) != hipSuccess) {
                    (void)hipEventDestroy(e0);
                    break;
                }
                float best_ms = 1e30f;
                for (int c = 0; c < found; ++c) {
                    if (hipblasLtMatmul(h, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &res[c].algo, ws, ws_bytes,
                                        stream) != HIPBLAS_STATUS_SUCCESS)
                        continue;
                    (void)hipEventRecord(e0, stream);
                    bool ok = true;
                    for (int r = 0; r < 3 && ok; ++r)
                        ok = hipblasLtMatmul(h, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &res[c].algo, ws,
                                             ws_bytes, stream) == HIPBLAS_STATUS_SUCCESS;
                    (void)hipEventRecord(e1, stream);
                    float ms = 0.f;
                    if (ok && hipEventSynchronize(e1) == hipSuccess && hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
                        ms < best_ms)
                        best_ms = ms, best = c;
                }
                (void)hipEventDestroy(e0);
                (void)hipEventDestroy(e1);
            }
            algo = res[best].algo;
            std::lock_guard<std::mutex> lock(g_lt_mutex);
            g_algo_cache[key] = algo;
        }
        if (hipblasLtMatmul(h, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &algo, ws, ws_bytes, stream) !=
            HIPBLAS_STATUS_SUCCESS)
            break;
        rc = DLRM_OK;
    } while (false);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (ld) hipblasLtMatrixLayoutDestroy(ld);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (desc) hipblasLtMatmulDescDestroy(desc);
    return rc;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Slices of the batch dimension for the weight-gradient GEMM (its K dimension is M): enough
// output tiles for the chip when N x K is small, and a fixed split for a given M.
constexpr int kMaxSplit = 8;
constexpr int64_t kSplitRows = 2048;
int dw_split(int64_t M) {
    int s = 1;
    while (s < kMaxSplit && M % (2 * s) == 0 && M / (2 * s) >= kSplitRows) s *= 2;
    return s;
}

// The two sums that end a layer's backward, in one launch.  Blocks [0, ncb): the bias gradient,
// db[c] = sum over the row blocks of partial[blk][c], one column per wavefront (four per block).
// Blocks past them: the weight gradient, dW[i] = sum over s of part[s][i] (slices in order, all S
// loaded before the first add), 256 elements per block; none when S == 1 (the GEMM wrote dW).
__global__ __launch_bounds__(256) void k_grad_sums(const float *__restrict__ partial, int32_t nblk, int32_t N,
                                                   float *__restrict__ db, uint32_t ncb,
                                                   const float *__restrict__ part, int32_t S, int64_t n,
                                                   float *__restrict__ dW) {
    if (blockIdx.x < ncb) {  // block-uniform
        const int32_t c = blockIdx.x * 4 + static_cast<int32_t>(wave_id());
        if (c >= N) return;  // wave-uniform
        const float s = wave_colsum(partial, nblk, N, c);
        if ((threadIdx.x & 63) == 0) db[c] = s;
        return;
    }
    const int64_t i = static_cast<int64_t>(blockIdx.x - ncb) * 256 + threadIdx.x;
    if (i >= n) return;
    float v[kMaxSplit];
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q) v[q] = part[static_cast<uint64_t>(min(q, S - 1)) * n + i];
    float s = v[0];
#pragma unroll
    for (int q = 1; q < kMaxSplit; ++q)
        if (q < S) s += v[q];
    dW[i] = s;
}

bool layer_dims_ok(int64_t M, int32_t N, int32_t K) {
    return M >= 1 && M < (int64_t(1) << 31) && N >= 1 && K >= 1 && N <= 65536 && K <= 65536 && N % 8 == 0 &&
           K % 8 == 0;
}

}  // namespace
}  // namespace dlrm

using namespace dlrm;

// Workspace: [GEMM scratch][bias-gradient partials][split-K partials of dW].
inline size_t partials_bytes(int64_t M, int32_t N) {
    return align_up(static_cast<size_t>((M + kGradRows - 1) / kGradRows) * static_cast<size_t>(N) * 4, 256);
}

extern "C" size_t dlrm_linear_workspace_size(int64_t M, int32_t N, int32_t K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    const int S = dw_split(M);
    return kGemmScratch + partials_bytes(M, N) +
           (S > 1 ? align_up(static_cast<size_t>(S) * N * static_cast<size_t>(K) * 4, 256) : 0);
}

extern "C" int dlrm_linear_fwd(const uint16_t *x, const uint16_t *W, const float *b, int64_t M, int32_t N,
                               int32_t K, int32_t act, void *y, int32_t y_dtype, void *workspace,
                               size_t workspace_bytes, dlrm_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!layer_dims_ok(M, N, K)) return M >= 1 && N >= 1 && K >= 1 ? DLRM_ERR_UNSUPPORTED : DLRM_ERR_INVALID_ARG;
    if (act != DLRM_ACT_NONE && act != DLRM_ACT_RELU) return DLRM_ERR_INVALID_ARG;
    if (y_dtype != DLRM_F32 && y_dtype != DLRM_BF16) return DLRM_ERR_INVALID_ARG;
    if (!x || !W || !b || !y || !aligned(x, 16) || !aligned(W, 16) || !aligned(b, 4) || !aligned(y, 16))
        return DLRM_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < dlrm_linear_workspace_size(M, N, K))
        return DLRM_ERR_WORKSPACE;
    // row-major y[M][N] = x[M][K] W[N][K]^T  <=>  column-major y^T (N x M) = W^T x^T
    int rc = lt_gemm(stream, true, false, N, M, K, W, K, x, K, y, y_dtype == DLRM_F32 ? HIP_R_32F : HIP_R_16BF, b,
                     act == DLRM_ACT_RELU, workspace, kGemmScratch);
    if (rc != DLRM_OK) return rc;
    return launch_status();
}

extern "C" int dlrm_linear_bwd(const float *dy, const void *y, int32_t y_dtype, int32_t act, const uint16_t *x,
                               const uint16_t *W, int64_t M, int32_t N, int32_t K, uint16_t *dz_bf16, float *dx,
                               float *dW, float *db, void *workspace, size_t workspace_bytes,
                               dlrm_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!layer_dims_ok(M, N, K)) return M >= 1 && N >= 1 && K >= 1 ? DLRM_ERR_UNSUPPORTED : DLRM_ERR_INVALID_ARG;
    if (act != DLRM_ACT_NONE && act != DLRM_ACT_RELU) return DLRM_ERR_INVALID_ARG;
    if (y_dtype != DLRM_F32 && y_dtype != DLRM_BF16) return DLRM_ERR_INVALID_ARG;
    if (!dy || !x || !W || !dz_bf16 || !dW || !db || (act == DLRM_ACT_RELU && !y)) return DLRM_ERR_INVALID_ARG;
    if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(W, 16) || !aligned(dz_bf16, 16) || !aligned(dW, 16) ||
        !aligned(db, 4) || (dx && !aligned(dx, 16)) || (y && !aligned(y, 16)))
        return DLRM_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < dlrm_linear_workspace_size(M, N, K))
        return DLRM_ERR_WORKSPACE;
    float *partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + kGemmScratch);
    const int32_t nblk = static_cast<int32_t>((M + kGradRows - 1) / kGradRows);
    const dim3 grid(nblk, (N + 1023) / 1024);
    if (act == DLRM_ACT_RELU) {
        if (y_dtype == DLRM_F32)
            DLRM_LAUNCH("relu_grad", (k_relu_grad<true, DLRM_F32>), grid, dim3(256), 0, stream, dy, y, M, N, dz_bf16, partial);
        else
            DLRM_LAUNCH("relu_grad", (k_relu_grad<true, DLRM_BF16>), grid, dim3(256), 0, stream, dy, y, M, N, dz_bf16, partial);
    } else {
        DLRM_LAUNCH("relu_grad", (k_relu_grad<false, DLRM_F32>), grid, dim3(256), 0, stream, dy, y, M, N, dz_bf16, partial);
    }
    if (hipGetLastError() != hipSuccess) return DLRM_ERR_HIP;
    int rc;
    if (dx) {
        // row-major dx[M][K] = dz[M][N] W[N][K]  <=>  column-major dx^T (K x M) = W^T(K x N, stored as W) dz^T
        rc = lt_gemm(stream, false, false, K, M, N, W, K, dz_bf16, N, dx, HIP_R_32F, nullptr, false, workspace,
                     kGemmScratch);
        if (rc != DLRM_OK) return rc;
    }
    // row-major dW[N][K] = dz^T x  <=>  column-major dW^T (K x N) = x^T(K x M, stored as x) dz (M x N);
    // split over S slices of the rows (a strided batch), then the slices summed in order
    const int S = dw_split(M);
    float *part = nullptr;
    if (S == 1) {
        rc = lt_gemm(stream, false, true, K, N, M, x, K, dz_bf16, N, dW, HIP_R_32F, nullptr, false, workspace,
                     kGemmScratch);
    } else {
        const int64_t Ms = M / S;
        part = reinterpret_cast<float *>(static_cast<char *>(workspace) + kGemmScratch + partials_bytes(M, N));
        rc = lt_gemm(stream, false, true, K, N, Ms, x, K, dz_bf16, N, part, HIP_R_32F, nullptr, false, workspace,
                     kGemmScratch, S, Ms * K, Ms * N, static_cast<int64_t>(K) * N);
    }
    if (rc != DLRM_OK) return rc;
    // the bias gradient's column sums and (split GEMM) the sum of the slices
    const uint32_t ncb = static_cast<uint32_t>((N + 3) / 4);
    const int64_t n = S > 1 ? static_cast<int64_t>(K) * N : 0;
    DLRM_LAUNCH("grad_sums", k_grad_sums, dim3(ncb + static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream,
                partial, nblk, N, db, ncb, part, S, n, dW);
    return launch_status();
}

extern "C" size_t dlrm_bce_head_workspace_size(int64_t M, int32_t K) {
    if (M < 1 || K < 1 || K > kHeadMaxK) return 0;
    return align_up(static_cast<size_t>(kHeadBlocks) * (K + 2) * 4, 256);
}

extern "C" int dlrm_bce_head(const uint16_t *x, const uint16_t *w, const float *b, const float *t, int64_t M,
                             int32_t K, float *p, float *loss, float *dx, float *dw, float *db, void *workspace,
                             size_t workspace_bytes, dlrm_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (M < 1 || K < 1) return DLRM_ERR_INVALID_ARG;
    if (K > kHeadMaxK || K % 8 != 0 || M >= (int64_t(1) << 31)) return DLRM_ERR_UNSUPPORTED;
    if (!x || !w || !b || !t || !p || !loss || !dx || !dw || !db) return DLRM_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(dx, 16)) return DLRM_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < dlrm_bce_head_workspace_size(M, K))
        return DLRM_ERR_WORKSPACE;
    float *partial = static_cast<float *>(workspace);
    if (K <= 64)
        DLRM_LAUNCH("bce_head", k_bce_head<1>, dim3(kHeadBlocks), dim3(256), 0, stream, x, w, b, t, M, K, p, dx, partial);
    else if (K <= 128)
        DLRM_LAUNCH("bce_head", k_bce_head<2>, dim3(kHeadBlocks), dim3(256), 0, stream, x, w, b, t, M, K, p, dx, partial);
    else if (K <= 256)
        DLRM_LAUNCH("bce_head", k_bce_head<4>, dim3(kHeadBlocks), dim3(256), 0, stream, x, w, b, t, M, K, p, dx, partial);
    else if (K <= 512)
        DLRM_LAUNCH("bce_head", k_bce_head<8>, dim3(kHeadBlocks), dim3(256), 0, stream, x, w, b, t, M, K, p, dx, partial);
    else
        DLRM_LAUNCH("bce_head", k_bce_head<16>, dim3(kHeadBlocks), dim3(256), 0, stream, x, w, b, t, M, K, p, dx, partial);
    DLRM_LAUNCH("bce_final", k_bce_final, dim3((K + 2 + 3) / 4), dim3(256), 0, stream, partial, kHeadBlocks, K, M,
                dw, db, loss);
    return launch_status();
}

extern "C" int dlrm_sgd_dense(float *w32, uint16_t *w16, const float *g, int64_t n, float lr,
                              dlrm_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (n < 0) return DLRM_ERR_INVALID_ARG;
    if (n == 0) return DLRM_OK;
    if (!w32 || !g) return DLRM_ERR_INVALID_ARG;
    DLRM_LAUNCH("sgd_dense", k_sgd_dense, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream, w32, w16, g,
                n, lr);
    return launch_status();
}

extern "C" int dlrm_sgd_dense_multi(int32_t count, float *const *w32, uint16_t *const *w16, const float *const *g,
                                    const int64_t *n, float lr, dlrm_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (count < 0 || count > kSgdMaxTensors) return DLRM_ERR_INVALID_ARG;
    if (count == 0) return DLRM_OK;
    if (!w32 || !g || !n) return DLRM_ERR_INVALID_ARG;
    SgdMulti a{};
    uint64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        if (n[i] < 0 || (n[i] > 0 && (!w32[i] || !g[i]))) return DLRM_ERR_INVALID_ARG;
        a.w32[i] = w32[i];
        a.w16[i] = w16 ? w16[i] : nullptr;
        a.g[i] = g[i];
        a.n[i] = n[i];
        a.boff[i] = static_cast<uint32_t>(blocks);
        blocks += (static_cast<uint64_t>(n[i]) + kSgdPerBlock - 1) / kSgdPerBlock;
        if (blocks >= (uint64_t(1) << 31)) return DLRM_ERR_UNSUPPORTED;
    }
    a.boff[count] = static_cast<uint32_t>(blocks);
    a.count = count;
    a.lr = lr;
    if (blocks == 0) return DLRM_OK;
    DLRM_LAUNCH("sgd_dense_multi", k_sgd_dense_multi, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, a);
    return launch_status();
}

extern "C" int dlrm_cast_rows(const void *src, int32_t src_dtype, int64_t src_ld, int64_t M, int32_t cols, void *dst,
                              int32_t dst_dtype, int32_t dst_cols, dlrm_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if ((src_dtype != DLRM_F32 && src_dtype != DLRM_BF16) || (dst_dtype != DLRM_F32 && dst_dtype != DLRM_BF16))
        return DLRM_ERR_INVALID_ARG;
    if (M < 0 || cols < 0 || dst_cols < cols || src_ld < cols) return DLRM_ERR_INVALID_ARG;
    const int64_t total = M * dst_cols;
    if (total == 0) return DLRM_OK;
    if (!src || !dst || total >= (int64_t(1) << 40)) return DLRM_ERR_INVALID_ARG;
    const int rpl = cast_rows_per_lane(dst_cols);
    const int64_t rows_per_block = static_cast<int64_t>(256 / cast_groups(dst_cols)) * rpl;
    const int64_t row_blocks = (M + rows_per_block - 1) / rows_per_block;
    if (row_blocks >= (int64_t(1) << 31)) return DLRM_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<uint32_t>(row_blocks), static_cast<uint32_t>((dst_cols + 1023) / 1024));
    const bool vec = dst_cols % 4 == 0 && aligned(dst, 16);
    auto go = [&](auto st, auto dt) {
        constexpr int ST = decltype(st)::value, DT = decltype(dt)::value;
        if (vec)
            DLRM_LAUNCH("cast_rows", (k_cast_rows<ST, DT, true>), grid, dim3(256), 0, stream, src, src_ld, M, cols,
                        dst, dst_cols, rpl);
        else
            DLRM_LAUNCH("cast_rows", (k_cast_rows<ST, DT, false>), grid, dim3(256), 0, stream, src, src_ld, M, cols,
                        dst, dst_cols, rpl);
    };
    using F = std::integral_constant<int, DLRM_F32>;
    using H = std::integral_constant<int, DLRM_BF16>;
    if (src_dtype == DLRM_F32 && dst_dtype == DLRM_BF16) go(F{}, H{});
    else if (src_dtype == DLRM_F32) go(F{}, F{});
    else if (dst_dtype == DLRM_BF16) go(H{}, H{});
    else go(H{}, F{});
    return launch_status();
}
