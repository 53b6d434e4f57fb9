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

__device__ __forceinline__ uint64_t lanemask_lt() {
    const uint32_t lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------- host helpers

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
                       int32_t dtype, const int64_t *indices, const int64_t *offsets,
                       const float *weights, int64_t B, int64_t nnz) {
    if (T < 1 || T > kMaxTables || D < 1 || B < 0 || nnz < 0) return DLRM_ERR_INVALID_ARG;
    if (dtype != DLRM_F32 && dtype != DLRM_BF16) return DLRM_ERR_INVALID_ARG;
    if (D > 512 || (D * elem_size(dtype)) % 16 != 0) return DLRM_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(T) * B >= (int64_t(1) << 31) || nnz >= (int64_t(1) << 31))
        return DLRM_ERR_UNSUPPORTED;
    if (!tables || !rows || !offsets) return DLRM_ERR_INVALID_ARG;
    if (nnz > 0 && !indices) return DLRM_ERR_INVALID_ARG;
    if (!aligned(offsets, 8) || (indices && !aligned(indices, 8)) || (weights && !aligned(weights, 4)))
        return DLRM_ERR_INVALID_ARG;
    for (int t = 0; t < T; ++t) {
        if (rows[t] < 1) return DLRM_ERR_INVALID_ARG;
        if (!tables[t] || !aligned(tables[t], 16)) return DLRM_ERR_INVALID_ARG;
    }
    return DLRM_OK;
}

}  // namespace dlrm
