// Embedding-bag lookup with sum / weighted-sum pooling (the lookup stage of the DLRM forward
// pass: robocikowo.com "DLRM", paragraph "Forward pass", stage (2), and its paragraph on the
// embedding tables E_i: V_i x D).
//
// The operation is a gather of random table rows, so it is bound by HBM latency and bandwidth.
// Design for gfx950:
//   - A row is D*s bytes = G chunks of 16 bytes; a lane group of G lanes covers one row with
//     one 16-byte load per lane (global_load_dwordx4), so every row read is fully coalesced.
//   - Multi-hot bags: one wavefront per bag at a time (4 consecutive bags per wave, in turn).
//     The wave loads up to 64 of the bag's indices with one coalesced load, broadcasts them
//     with cross-lane permutes, and its 64/G lane groups each issue U row loads before the
//     first use, so 64/G*U rows of the bag are in flight at once.  Group partial sums are
//     combined in a fixed butterfly.
//   - One-hot / short bags: each lane group owns BPG bags and issues the first row of all of
//     them before accumulating.
//   - Blocks are remapped so each XCD walks a contiguous range of bags; bags are table-major,
//     so each XCD's L2 serves about T/8 tables and keeps more of their hot rows.
//   - fp32 accumulation in a fixed order: results are bitwise reproducible; a bag of one row
//     returns that row exactly.
#include "common.h"
#include "pool.h"

namespace dlrm {
namespace {

// Bags per wavefront in the multi-hot lookup: a wave walks 4 consecutive bags (of one table,
// mostly) in turn, which measured 4% faster than one bag per wave (fewer, longer waves).
constexpr int kPoolBagsPerWave = 4;

struct PoolArgs {
    const char *tables[kMaxTables];
    const void *indices;  // int64 or int32 (the kernel's IT)
    const void *offsets;  // same type as the indices
    const float *weights;
    void *out;            // fp32 or bf16 (the kernel's OT)
    uint32_t B;
    uint32_t nbags;
    int32_t T;
    int32_t D;
    uint32_t row_bytes;
    uint32_t nblocks;  // blocks launched (a multiple of 8)
};

// One wavefront per bag at a time (multi-hot), kPoolBagsPerWave bags per wave.  G lanes per row,
// NG = 64/G groups, U rows per group in flight.
template <int DT, int G, bool WEIGHTED, typename IT, int OT>
__global__ __launch_bounds__(256) void k_pool_wave_per_bag(PoolArgs a) {
    const IT *indices = static_cast<const IT *>(a.indices);
    const IT *offsets = static_cast<const IT *>(a.offsets);
    constexpr int NG = kWave / G;
    constexpr int EPC = Elem<DT>::kPerChunk;
    // rows per lane group in flight: with weights, 8 took 73 registers (6 waves per SIMD) and
    // 4 keeps 8 waves (weighted multi-hot lookup 309 -> 278 us); without, 4, 6 and 8 measure alike
    constexpr int U = WEIGHTED ? 4 : 8;
    const uint32_t lb = xcd_contiguous(blockIdx.x, a.nblocks);
    const uint32_t bag0 = (lb * 4 + wave_id()) * kPoolBagsPerWave;
    const int lane = threadIdx.x & 63;
    const int grp = lane / G, c = lane % G;
    for (uint32_t bag = bag0; bag < min(bag0 + kPoolBagsPerWave, a.nbags); ++bag) {  // wave-uniform
        const uint32_t t = bag / a.B, b = bag - t * a.B;
        const char *tab = a.tables[t] + c * 16;
        const int64_t start = offsets[bag], end = offsets[bag + 1];

        float acc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
        for (int64_t base = start; base < end; base += kWave) {
            const int n = static_cast<int>(min<int64_t>(kWave, end - base));
            const int64_t my_idx = lane < n ? static_cast<int64_t>(indices[base + lane]) : 0;
            float my_w = 1.f;
            if constexpr (WEIGHTED) my_w = lane < n ? a.weights[base + lane] : 0.f;
            for (int r0 = 0; r0 < n; r0 += NG * U) {
                uint4 v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int r = r0 + u * NG + grp;
                    const int64_t idx = __shfl(my_idx, r < n ? r : 0);
                    v[u] = r < n ? load_row_chunk(tab, idx, a.row_bytes) : make_uint4(0, 0, 0, 0);
                }
                // the weights are fetched from their lanes only now, while the rows are in flight
                if constexpr (WEIGHTED) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int r = r0 + u * NG + grp;
                    const float w = WEIGHTED ? __shfl(my_w, r < n ? r : 0) : 1.f;
                    if (r < n) accumulate<DT, WEIGHTED>(acc, v[u], w);
                }
            }
        }
        // combine the NG group partials (fixed butterfly: every group ends with identical bits)
#pragma unroll
        for (int s = G; s < kWave; s <<= 1)
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], s);
        if (grp == 0) store_pooled<DT, OT>(a.out, (static_cast<uint64_t>(b) * a.T + t) * a.D + c * EPC, acc);
    }
}

// One lane group per bag (one-hot or short bags); each group owns BPG bags.
template <int DT, int G, bool WEIGHTED, int BPG, typename IT, int OT>
__global__ __launch_bounds__(256) void k_pool_group_per_bag(PoolArgs a) {
    const IT *indices = static_cast<const IT *>(a.indices);
    const IT *offsets = static_cast<const IT *>(a.offsets);
    constexpr int NG = kWave / G;
    constexpr int EPC = Elem<DT>::kPerChunk;
    const uint32_t lb = xcd_contiguous(blockIdx.x, a.nblocks);
    const uint32_t wave = lb * 4 + wave_id();
    const int lane = threadIdx.x & 63;
    const int grp = lane / G, c = lane % G;
    const uint32_t bag0 = wave * (NG * BPG) + grp;

    int64_t s[BPG], e[BPG];
    const char *tab[BPG];
#pragma unroll
    for (int k = 0; k < BPG; ++k) {
        const uint32_t bag = bag0 + k * NG;
        const bool ok = bag < a.nbags;
        s[k] = ok ? static_cast<int64_t>(offsets[bag]) : 0;
        e[k] = ok ? static_cast<int64_t>(offsets[bag + 1]) : 0;
        tab[k] = a.tables[ok ? bag / a.B : 0] + c * 16;
    }
    float acc[BPG][EPC];
#pragma unroll
    for (int k = 0; k < BPG; ++k)
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[k][q] = 0.f;

    // first row of every bag: BPG row loads in flight per lane
    {
        int64_t idx[BPG];
        float w[BPG];
#pragma unroll
        for (int k = 0; k < BPG; ++k) {
            idx[k] = s[k] < e[k] ? static_cast<int64_t>(indices[s[k]]) : 0;
            w[k] = (WEIGHTED && s[k] < e[k]) ? a.weights[s[k]] : 1.f;
        }
        uint4 v[BPG];
#pragma unroll
        for (int k = 0; k < BPG; ++k)
            v[k] = s[k] < e[k] ? load_row_chunk(tab[k], idx[k], a.row_bytes) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < BPG; ++k)
            if (s[k] < e[k]) accumulate<DT, WEIGHTED>(acc[k], v[k], w[k]);
    }
    // remaining rows, four in flight
#pragma unroll
    for (int k = 0; k < BPG; ++k) {
        for (int64_t j = s[k] + 1; j < e[k]; j += 4) {
            uint4 v[4];
            float w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = j + u < e[k];
                const int64_t idx = ok ? static_cast<int64_t>(indices[j + u]) : 0;
                w[u] = (WEIGHTED && ok) ? a.weights[j + u] : 1.f;
                v[u] = ok ? load_row_chunk(tab[k], idx, a.row_bytes) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (j + u < e[k]) accumulate<DT, WEIGHTED>(acc[k], v[u], w[u]);
        }
    }
#pragma unroll
    for (int k = 0; k < BPG; ++k) {
        const uint32_t bag = bag0 + k * NG;
        if (bag < a.nbags) {
            const uint32_t t = bag / a.B, b = bag - t * a.B;
            store_pooled<DT, OT>(a.out, (static_cast<uint64_t>(b) * a.T + t) * a.D + c * EPC, acc[k]);
        }
    }
}

// Any row width: one thread per (bag, 16-byte chunk).
template <int DT, bool WEIGHTED, typename IT, int OT>
__global__ __launch_bounds__(256) void k_pool_generic(PoolArgs a, uint32_t chunks) {
    const IT *indices = static_cast<const IT *>(a.indices);
    const IT *offsets = static_cast<const IT *>(a.offsets);
    constexpr int EPC = Elem<DT>::kPerChunk;
    const uint64_t gid = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const uint64_t bag = gid / chunks;
    if (bag >= a.nbags) return;
    const uint32_t c = static_cast<uint32_t>(gid % chunks);
    const uint32_t t = static_cast<uint32_t>(bag / a.B), b = static_cast<uint32_t>(bag - uint64_t(t) * a.B);
    const char *tab = a.tables[t] + c * 16;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    const int64_t j1 = offsets[bag + 1];
    for (int64_t j = offsets[bag]; j < j1; ++j) {
        const float w = WEIGHTED ? a.weights[j] : 1.f;
        accumulate<DT, WEIGHTED>(acc, load_row_chunk(tab, static_cast<int64_t>(indices[j]), a.row_bytes), w);
    }
    store_pooled<DT, OT>(a.out, (static_cast<uint64_t>(b) * a.T + t) * a.D + c * EPC, acc);
}

// ---------------------------------------------------------------- index / offset check

struct CheckArgs {
    int64_t rows[kMaxTables];
    const void *indices;
    const void *offsets;
    uint32_t B;
    uint32_t nbags;
    int64_t nnz;
    int *flag;
};

__global__ void k_set_int(int *p, int v) { *p = v; }

template <typename IT>
__global__ __launch_bounds__(256) void k_check_csr(CheckArgs a) {
    const IT *indices = static_cast<const IT *>(a.indices);
    const IT *offsets = static_cast<const IT *>(a.offsets);
    const uint64_t bag = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (a.nbags == 0) {
        if (bag == 0 && (offsets[0] != 0 || a.nnz != 0)) *a.flag = 1;
        return;
    }
    if (bag >= a.nbags) return;
    const int64_t o0 = offsets[bag], o1 = offsets[bag + 1];
    bool bad = o1 < o0 || o0 < 0 || o1 > a.nnz;
    if (bag == 0 && o0 != 0) bad = true;
    if (bag + 1 == a.nbags && o1 != a.nnz) bad = true;
    const int64_t V = a.rows[bag / a.B];
    const int64_t lo = max<int64_t>(o0, 0), hi = min<int64_t>(o1, a.nnz);
    for (int64_t j = lo; j < hi; ++j) {
        const int64_t i = indices[j];
        if (i < 0 || i >= V) bad = true;
    }
    if (bad) *a.flag = 1;
}

}  // namespace

// Runs the device-side CSR check; `flag` is 4 bytes of device scratch the caller lends.
int check_csr_on_device(const int64_t *rows, int32_t T, const void *indices, const void *offsets,
                        int32_t index_type, int64_t B, int64_t nnz, int *flag, hipStream_t stream) {
    CheckArgs c{};
    for (int t = 0; t < T; ++t) c.rows[t] = rows[t];
    c.indices = indices;
    c.offsets = offsets;
    c.B = static_cast<uint32_t>(B);
    c.nbags = static_cast<uint32_t>(T * B);
    c.nnz = nnz;
    c.flag = flag;
    DLRM_LAUNCH("set_int", k_set_int, dim3(1), dim3(1), 0, stream, flag, 0);
    const uint32_t blocks = c.nbags == 0 ? 1 : (c.nbags + 255) / 256;
    if (index_type == DLRM_INDEX_I32)
        DLRM_LAUNCH("check_csr", k_check_csr<int32_t>, dim3(blocks), dim3(256), 0, stream, c);
    else
        DLRM_LAUNCH("check_csr", k_check_csr<int64_t>, dim3(blocks), dim3(256), 0, stream, c);
    if (hipGetLastError() != hipSuccess) return DLRM_ERR_HIP;
    int host_flag = 0;
    if (hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return DLRM_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return DLRM_ERR_HIP;
    return host_flag ? DLRM_ERR_INDEX_RANGE : DLRM_OK;
}

namespace {

template <int DT, int G, bool W, typename IT, int OT>
void launch_pool(const PoolArgs &a0, bool wave_per_bag, hipStream_t stream) {
    PoolArgs a = a0;
    constexpr int NG = kWave / G;
    if (wave_per_bag) {
        a.nblocks = round_up_xcd((a.nbags + 4 * kPoolBagsPerWave - 1) / (4 * kPoolBagsPerWave));
        DLRM_LAUNCH("pool_wave_per_bag", (k_pool_wave_per_bag<DT, G, W, IT, OT>), dim3(a.nblocks), dim3(256), 0, stream, a);
    } else {
        constexpr int BPG = G >= 64 ? 1 : (G >= 32 ? 2 : 4);
        const uint64_t per_block = 4ull * NG * BPG;
        a.nblocks = round_up_xcd((a.nbags + per_block - 1) / per_block);
        DLRM_LAUNCH("pool_group_per_bag", (k_pool_group_per_bag<DT, G, W, BPG, IT, OT>), dim3(a.nblocks), dim3(256), 0,
                    stream, a);
    }
}

template <int DT, bool W, typename IT, int OT>
void dispatch_g(const PoolArgs &a, uint32_t chunks, bool wave_per_bag, hipStream_t stream) {
    switch (chunks) {
        case 4: launch_pool<DT, 4, W, IT, OT>(a, wave_per_bag, stream); break;
        case 8: launch_pool<DT, 8, W, IT, OT>(a, wave_per_bag, stream); break;
        case 16: launch_pool<DT, 16, W, IT, OT>(a, wave_per_bag, stream); break;
        case 32: launch_pool<DT, 32, W, IT, OT>(a, wave_per_bag, stream); break;
        case 64: launch_pool<DT, 64, W, IT, OT>(a, wave_per_bag, stream); break;
        default: {
            const uint64_t threads = static_cast<uint64_t>(a.nbags) * chunks;
            DLRM_LAUNCH("pool_generic", (k_pool_generic<DT, W, IT, OT>), dim3((threads + 255) / 256), dim3(256), 0,
                        stream, a, chunks);
        }
    }
}

template <typename IT, int OT>
void dispatch_pool(const PoolArgs &a, int32_t dtype, uint32_t chunks, bool wave_per_bag, bool weighted,
                   hipStream_t stream) {
    if (dtype == DLRM_F32) {
        if (weighted) dispatch_g<DLRM_F32, true, IT, OT>(a, chunks, wave_per_bag, stream);
        else dispatch_g<DLRM_F32, false, IT, OT>(a, chunks, wave_per_bag, stream);
    } else {
        if (weighted) dispatch_g<DLRM_BF16, true, IT, OT>(a, chunks, wave_per_bag, stream);
        else dispatch_g<DLRM_BF16, false, IT, OT>(a, chunks, wave_per_bag, stream);
    }
}

}  // namespace
}  // namespace dlrm

extern "C" int emb_bag_fwd_ex(const void *const *tables, const int64_t *rows, int32_t T, int32_t D,
                              int32_t dtype, const void *indices, const void *offsets,
                              int32_t index_type, const float *per_sample_weights, int64_t B,
                              int64_t nnz, void *out, int32_t out_dtype, uint32_t flags,
                              dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (index_type != DLRM_INDEX_I64 && index_type != DLRM_INDEX_I32) return DLRM_ERR_INVALID_ARG;
    if (out_dtype != DLRM_F32 && out_dtype != DLRM_BF16) return DLRM_ERR_INVALID_ARG;
    int rc = check_batch(tables, rows, T, D, dtype, indices, offsets, index_type, per_sample_weights, B, nnz);
    if (rc != DLRM_OK) return rc;
    if (B > 0 && (!out || !aligned(out, 16))) return DLRM_ERR_INVALID_ARG;
    if (flags & ~DLRM_FLAG_CHECK_INDICES) return DLRM_ERR_INVALID_ARG;
    if (B == 0) {
        if (nnz != 0) return DLRM_ERR_INVALID_ARG;
        return DLRM_OK;
    }
    if (flags & DLRM_FLAG_CHECK_INDICES) {
        // the output buffer lends 4 bytes for the flag; it is overwritten below
        rc = check_csr_on_device(rows, T, indices, offsets, index_type, B, nnz, reinterpret_cast<int *>(out),
                                 stream);
        if (rc != DLRM_OK) return rc;
    }
    PoolArgs a{};
    for (int t = 0; t < T; ++t) a.tables[t] = static_cast<const char *>(tables[t]);
    a.indices = indices;
    a.offsets = offsets;
    a.weights = per_sample_weights;
    a.out = out;
    a.B = static_cast<uint32_t>(B);
    a.nbags = static_cast<uint32_t>(T * B);
    a.T = T;
    a.D = D;
    a.row_bytes = static_cast<uint32_t>(D * elem_size(dtype));
    const uint32_t chunks = a.row_bytes / 16;
    // multi-hot bags (4+ rows on average) get a whole wavefront each
    const bool wave_per_bag = nnz >= 4 * static_cast<int64_t>(a.nbags);
    const bool weighted = per_sample_weights != nullptr;
    if (index_type == DLRM_INDEX_I64) {
        if (out_dtype == DLRM_F32) dispatch_pool<int64_t, DLRM_F32>(a, dtype, chunks, wave_per_bag, weighted, stream);
        else dispatch_pool<int64_t, DLRM_BF16>(a, dtype, chunks, wave_per_bag, weighted, stream);
    } else {
        if (out_dtype == DLRM_F32) dispatch_pool<int32_t, DLRM_F32>(a, dtype, chunks, wave_per_bag, weighted, stream);
        else dispatch_pool<int32_t, DLRM_BF16>(a, dtype, chunks, wave_per_bag, weighted, stream);
    }
    return launch_status();
}

extern "C" int emb_bag_fwd(const void *const *tables, const int64_t *rows, int32_t T, int32_t D,
                           int32_t dtype, const int64_t *indices, const int64_t *offsets,
                           const float *per_sample_weights, int64_t B, int64_t nnz, float *out,
                           uint32_t flags, dlrm_stream_t stream) {
    return emb_bag_fwd_ex(tables, rows, T, D, dtype, indices, offsets, DLRM_INDEX_I64, per_sample_weights, B,
                          nnz, out, DLRM_F32, flags, stream);
}
