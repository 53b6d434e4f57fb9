// Device-side synthetic table fill: the counter-hash table contents of the package's seeded
// generator module (SplitMix64 output function, Steele, Lea & Flood 2014), written straight
// into HBM so that tables of tens to hundreds of GB need no host copy.  Input generation only.
#include "common.h"
#include "dlrm_synth.h"

namespace dlrm {
namespace {

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float hashed_value(uint32_t t, uint64_t r, uint32_t d, uint64_t seed,
                                              float scale) {
    const uint64_t c = (static_cast<uint64_t>(t) << 50) | (r << 12) | d;
    const uint64_t h = splitmix64(seed ^ splitmix64(c));
    const int32_t m = static_cast<int32_t>(h >> 40);               // 24 bits
    const float unit = static_cast<float>(2 * m - (1 << 24)) * 0x1p-24f;  // exact
    return unit * scale;                                               // one RN multiply
}

// one thread writes 16 bytes: 4 fp32 or 8 bf16 elements of one row
template <int DT>
__global__ __launch_bounds__(256) void k_fill(char *table, uint64_t rows, uint32_t D, uint32_t t,
                                              uint64_t seed, float scale) {
    constexpr int EPC = DT == DLRM_BF16 ? 8 : 4;
    const uint32_t chunks = D / EPC;
    const uint64_t total = rows * chunks;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<uint64_t>(gridDim.x) * blockDim.x) {
        const uint64_t r = i / chunks;
        const uint32_t d0 = static_cast<uint32_t>(i % chunks) * EPC;
        float x[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) x[e] = hashed_value(t, r, d0 + e, seed, scale);
        if constexpr (DT == DLRM_F32) {
            *reinterpret_cast<float4 *>(table + i * 16) = make_float4(x[0], x[1], x[2], x[3]);
        } else {
            uint32_t b[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = f32_to_bf16_rne(x[e]);
            *reinterpret_cast<uint4 *>(table + i * 16) =
                make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                           b[6] | (b[7] << 16));
        }
    }
}

}  // namespace
}  // namespace dlrm

extern "C" int dlrm_synth_fill_table(void *table, int32_t dtype, int64_t rows, int32_t D, int32_t t,
                                     uint64_t seed, float scale, dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!table || rows < 1 || D < 1 || t < 0 || t >= (1 << 14) || rows >= (int64_t(1) << 38))
        return DLRM_ERR_INVALID_ARG;
    if (dtype != DLRM_F32 && dtype != DLRM_BF16) return DLRM_ERR_INVALID_ARG;
    if (D >= 4096 || (D * elem_size(dtype)) % 16 != 0 || !aligned(table, 16)) return DLRM_ERR_INVALID_ARG;
    const uint64_t chunks = static_cast<uint64_t>(rows) * (D * elem_size(dtype) / 16);
    const uint64_t want = (chunks + 255) / 256;
    const uint32_t blocks = static_cast<uint32_t>(want < 256 * 64 ? want : 256 * 64);
    if (dtype == DLRM_F32)
        DLRM_LAUNCH("synth_fill", k_fill<DLRM_F32>, dim3(blocks), dim3(256), 0, stream,
                           static_cast<char *>(table), static_cast<uint64_t>(rows),
                           static_cast<uint32_t>(D), static_cast<uint32_t>(t), seed, scale);
    else
        DLRM_LAUNCH("synth_fill", k_fill<DLRM_BF16>, dim3(blocks), dim3(256), 0, stream,
                           static_cast<char *>(table), static_cast<uint64_t>(rows),
                           static_cast<uint32_t>(D), static_cast<uint32_t>(t), seed, scale);
    return launch_status();
}
