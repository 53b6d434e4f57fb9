// Shared device helpers and host-side checks for the DLRM sparse library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dlrm_sparse.h"

namespace dlrm {

constexpr int kWave = 64;
constexpr int kMaxTables = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Workgroups are handed to the XCDs round-robin (id % 8).  With a grid whose size is a
// multiple of 8, this maps hardware block `bid` to a logical block so that each XCD works
// on one contiguous eighth of the logical range (so its L2 sees one eighth of the tables).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t bid, uint32_t nblocks) {
    const uint32_t per = nblocks / kNumXcd;
    return (bid % kNumXcd) * per + bid / kNumXcd;
}

// Index of this wavefront in its block, as a wave-uniform (scalar) value: the compiler cannot see
// that threadIdx.x >> 6 is uniform, and would otherwise do per-sample address math per lane.
__device__ __forceinline__ uint32_t wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const uint32_t lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

typedef float floatx4 __attribute__((ext_vector_type(4)));  // MFMA 16x16 accumulator fragment

// Position of pair (i, j), i < j, in the row-major strict upper triangle of an N x N matrix.
__device__ __forceinline__ int triu_pos(int i, int j, int N) {
    return i * N - (i * (i + 1)) / 2 + (j - i - 1);
}

// Loads and stores through the global address space (pointers staged in LDS would otherwise be
// generic/flat, and flat loads also count against the LDS wait counter).
#define DLRM_GLOBAL __attribute__((address_space(1)))

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int WORDS>
__device__ __forceinline__ void gload_words(const void *p, uint32_t *w) {
    if constexpr (WORDS == 1) {
        w[0] = *(const DLRM_GLOBAL uint32_t *)p;
    } else if constexpr (WORDS == 2) {
        const u32x2 v = *(const DLRM_GLOBAL u32x2 *)p;
        w[0] = v.x, w[1] = v.y;
    } else {
        const DLRM_GLOBAL u32x4 *q = (const DLRM_GLOBAL u32x4 *)p;
#pragma unroll
        for (int i = 0; i < WORDS / 4; ++i) {
            const u32x4 v = q[i];
            w[4 * i] = v.x, w[4 * i + 1] = v.y, w[4 * i + 2] = v.z, w[4 * i + 3] = v.w;
        }
    }
}

template <int WORDS>
__device__ __forceinline__ void gstore_words(void *p, const uint32_t *w) {
    if constexpr (WORDS == 1) {
        *(DLRM_GLOBAL uint32_t *)p = w[0];
    } else if constexpr (WORDS == 2) {
        *(DLRM_GLOBAL u32x2 *)p = u32x2{w[0], w[1]};
    } else {
        DLRM_GLOBAL u32x4 *q = (DLRM_GLOBAL u32x4 *)p;
#pragma unroll
        for (int i = 0; i < WORDS / 4; ++i) q[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    }
}

// ---------------------------------------------------------------- host helpers

// Kernel timing (trace.cpp): when enabled, each launch is bracketed by HIP events.
bool trace_on();
void trace_begin(hipStream_t s);
void trace_end(const char *name, hipStream_t s);

#define DLRM_LAUNCH(NAME, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                     \
    do {                                                                             \
        const bool dlrm_traced_ = ::dlrm::trace_on();                                \
        if (dlrm_traced_) ::dlrm::trace_begin(STREAM);                               \
        hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);          \
        if (dlrm_traced_) ::dlrm::trace_end(NAME, STREAM);                           \
    } while (0)

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int elem_size(int32_t dtype) { return dtype == DLRM_BF16 ? 2 : 4; }

inline uint32_t round_up_xcd(uint64_t blocks) {
    return static_cast<uint32_t>((blocks + kNumXcd - 1) / kNumXcd * kNumXcd);
}

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? DLRM_OK : DLRM_ERR_HIP;
}

// Shared validation of the CSR batch description (host side, no device access).
inline int check_batch(const void *const *tables, const int64_t *rows, int32_t T, int32_t D,
                       int32_t dtype, const void *indices, const void *offsets, int32_t index_type,
                       const float *weights, int64_t B, int64_t nnz) {
    const uintptr_t ib = index_type == DLRM_INDEX_I32 ? 4 : 8;
    if (T < 1 || T > kMaxTables || D < 1 || B < 0 || nnz < 0) return DLRM_ERR_INVALID_ARG;
    if (dtype != DLRM_F32 && dtype != DLRM_BF16) return DLRM_ERR_INVALID_ARG;
    if (D > 512 || (D * elem_size(dtype)) % 16 != 0) return DLRM_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(T) * B >= (int64_t(1) << 31) || nnz >= (int64_t(1) << 31))
        return DLRM_ERR_UNSUPPORTED;
    if (!tables || !rows || !offsets) return DLRM_ERR_INVALID_ARG;
    if (nnz > 0 && !indices) return DLRM_ERR_INVALID_ARG;
    if (!aligned(offsets, ib) || (indices && !aligned(indices, ib)) || (weights && !aligned(weights, 4)))
        return DLRM_ERR_INVALID_ARG;
    for (int t = 0; t < T; ++t) {
        if (rows[t] < 1) return DLRM_ERR_INVALID_ARG;
        if (!tables[t] || !aligned(tables[t], 16)) return DLRM_ERR_INVALID_ARG;
    }
    return DLRM_OK;
}

}  // namespace dlrm
