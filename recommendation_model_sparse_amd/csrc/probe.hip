// HBM read probes: a streaming read and a row gather with no output, the two read ceilings the
// lookup runs against on the running GPU (measurement context; no part of the method).
#include "common.h"
#include "dlrm_probe.h"

namespace dlrm {
namespace {

constexpr int kProbeBlocks = 4096;  // 16 workgroups per CU: enough loads in flight to saturate HBM

// Grid-stride streaming read: each thread keeps 4 16-byte loads in flight per round.
__global__ __launch_bounds__(256) void k_probe_read(const uint4 *__restrict__ buf, uint64_t n16,
                                                    uint32_t *__restrict__ sink) {
    constexpr int R = 4;
    __shared__ uint32_t red[4];
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint32_t acc = 0;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (R - 1) * stride < n16; i += R * stride) {
        uint4 v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = buf[i + r * stride];
#pragma unroll
        for (int r = 0; r < R; ++r) acc ^= v[r].x ^ v[r].y ^ v[r].z ^ v[r].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Row gather: a lane group of G = row_bytes/16 lanes reads a row with one 16-byte load per lane;
// each group keeps U rows in flight (indices loaded first, clamped into [0, rows)).
template <int G>
__global__ __launch_bounds__(256) void k_probe_gather(const char *__restrict__ buf, uint64_t rows,
                                                      const int64_t *__restrict__ idx, uint32_t n,
                                                      uint32_t *__restrict__ sink) {
    constexpr int U = 8;
    constexpr int NG = 256 / G;  // groups per block
    __shared__ uint32_t red[4];
    const int grp = threadIdx.x / G, c = threadIdx.x % G;
    const uint32_t groups = gridDim.x * NG;
    uint32_t acc = 0;
    for (uint32_t r0 = (blockIdx.x * NG + grp) * U; r0 < n; r0 += groups * U) {
        int64_t ix[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ix[u] = idx[min(r0 + u, n - 1)];
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t r = min(static_cast<uint64_t>(ix[u] < 0 ? 0 : ix[u]), rows - 1);
            v[u] = reinterpret_cast<const uint4 *>(buf + r * (G * 16))[c];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (r0 + u < n) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace
}  // namespace dlrm

extern "C" int dlrm_probe_read(const void *buf, uint64_t nbytes, uint32_t *sink, uint32_t sink_words,
                               dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!buf || !sink || sink_words < 1 || nbytes == 0 || nbytes % 16 != 0 || !aligned(buf, 16) ||
        !aligned(sink, 4))
        return DLRM_ERR_INVALID_ARG;
    const uint32_t blocks = sink_words < kProbeBlocks ? sink_words : kProbeBlocks;
    DLRM_LAUNCH("probe_read", k_probe_read, dim3(blocks), dim3(256), 0, stream, static_cast<const uint4 *>(buf),
                nbytes / 16, sink);
    return launch_status();
}

extern "C" int dlrm_probe_gather(const void *buf, int64_t rows, int32_t row_bytes, const int64_t *idx, int64_t n,
                                 uint32_t *sink, uint32_t sink_words, dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!buf || !sink || sink_words < 1 || rows < 1 || n < 0 || n >= (int64_t(1) << 31) || !aligned(buf, 16) ||
        !aligned(sink, 4) || row_bytes < 16 || row_bytes > 1024 || row_bytes % 16 != 0 || (n > 0 && !idx) ||
        (idx && !aligned(idx, 8)))
        return DLRM_ERR_INVALID_ARG;
    const int G = row_bytes / 16;
    if ((G & (G - 1)) != 0) return DLRM_ERR_INVALID_ARG;  // one row per power-of-two lane group
    if (n == 0) return DLRM_OK;
    const uint32_t blocks = sink_words < kProbeBlocks ? sink_words : kProbeBlocks;
    const char *b = static_cast<const char *>(buf);
    const uint32_t nn = static_cast<uint32_t>(n);
    const uint64_t r = static_cast<uint64_t>(rows);
    switch (G) {
        case 1: DLRM_LAUNCH("probe_gather", k_probe_gather<1>, dim3(blocks), dim3(256), 0, stream, b, r, idx, nn, sink); break;
        case 2: DLRM_LAUNCH("probe_gather", k_probe_gather<2>, dim3(blocks), dim3(256), 0, stream, b, r, idx, nn, sink); break;
        case 4: DLRM_LAUNCH("probe_gather", k_probe_gather<4>, dim3(blocks), dim3(256), 0, stream, b, r, idx, nn, sink); break;
        case 8: DLRM_LAUNCH("probe_gather", k_probe_gather<8>, dim3(blocks), dim3(256), 0, stream, b, r, idx, nn, sink); break;
        case 16: DLRM_LAUNCH("probe_gather", k_probe_gather<16>, dim3(blocks), dim3(256), 0, stream, b, r, idx, nn, sink); break;
        case 32: DLRM_LAUNCH("probe_gather", k_probe_gather<32>, dim3(blocks), dim3(256), 0, stream, b, r, idx, nn, sink); break;
        default: DLRM_LAUNCH("probe_gather", k_probe_gather<64>, dim3(blocks), dim3(256), 0, stream, b, r, idx, nn, sink); break;
    }
    return launch_status();
}
