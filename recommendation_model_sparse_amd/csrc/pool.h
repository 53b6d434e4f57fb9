// Row-gather helpers shared by the pooling kernels (emb_bag_fwd.hip, emb_interact_fwd.hip).
#pragma once

#include "common.h"

namespace dlrm {

template <int DT>
struct Elem;
template <>
struct Elem<DLRM_F32> {
    static constexpr int kPerChunk = 4;
};
template <>
struct Elem<DLRM_BF16> {
    static constexpr int kPerChunk = 8;
};

// acc += w * (16-byte chunk widened to fp32)
template <int DT, bool WEIGHTED>
__device__ __forceinline__ void accumulate(float *acc, const uint4 &v, float w) {
    if constexpr (DT == DLRM_F32) {
        const float x[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                            __uint_as_float(v.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = WEIGHTED ? fmaf(w, x[e], acc[e]) : acc[e] + x[e];
    } else {
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = bf16_lo(q[e]), hi = bf16_hi(q[e]);
            acc[2 * e] = WEIGHTED ? fmaf(w, lo, acc[2 * e]) : acc[2 * e] + lo;
            acc[2 * e + 1] = WEIGHTED ? fmaf(w, hi, acc[2 * e + 1]) : acc[2 * e + 1] + hi;
        }
    }
}

template <int DT>
__device__ __forceinline__ void store_chunk(float *dst, const float *acc) {
    constexpr int EPC = Elem<DT>::kPerChunk;
#pragma unroll
    for (int e = 0; e < EPC; e += 4)
        *reinterpret_cast<float4 *>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
}

// The pooled output of one lane: EPC consecutive values as fp32, or rounded to bf16 (nearest
// even, v_cvt_pk_bf16_f32), at element `elem` of the output.
template <int DT, int OT>
__device__ __forceinline__ void store_pooled(void *out, uint64_t elem, const float *acc) {
    constexpr int EPC = Elem<DT>::kPerChunk;
    if constexpr (OT == DLRM_F32) {
        store_chunk<DT>(static_cast<float *>(out) + elem, acc);
    } else {
        uint32_t w[EPC / 2];
#pragma unroll
        for (int e = 0; e < EPC / 2; ++e) {
            const __bf16 lo = static_cast<__bf16>(acc[2 * e]), hi = static_cast<__bf16>(acc[2 * e + 1]);
            w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        uint16_t *dst = static_cast<uint16_t *>(out) + elem;
        if constexpr (EPC == 8) *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        else *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    }
}

__device__ __forceinline__ uint4 load_row_chunk(const char *tab, int64_t idx, uint32_t row_bytes) {
    return *reinterpret_cast<const uint4 *>(tab + static_cast<uint64_t>(idx) * row_bytes);
}

}  // namespace dlrm
