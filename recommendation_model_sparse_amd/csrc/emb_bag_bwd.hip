// Embedding backward with row-wise Adagrad, in place (robocikowo.com "DLRM": the training
// sentence of the paragraph "Forward pass" names SGD/Adagrad; the lookup is linear in the
// table, so a row's gradient is the weighted sum of the pooled gradients of the bags that
// looked it up).
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   K4  expand: key_j = rowbase[t] + idx_j, val_j = j, bag_of[j] (one block per 256 bags,
//       offsets staged in LDS, binary search per position).
//   K5  stable LSD radix sort of (key, position), 8-bit digits, ceil(bits(sum V - 1)/8) passes.
//       Per pass: per-tile digit histograms, a per-digit scan across tiles, and a scatter that
//       ranks each key inside its tile with wavefront ballots (stable: ties keep order).
//   K6  unique keys and segment offsets (flag = key differs from its predecessor; a scan of
//       the flags), written only when the caller asks for them.
//   K7  chunked segment reduction fused with the update.  The sorted sequence is cut into
//       chunks of G positions; a lane group walks its chunk in order, summing
//       w * grad_pooled[bag] rows (one lane per 1..8 columns).  A segment that lies inside
//       one chunk is finished on the spot: row-wise Adagrad on the prefetched table row and
//       state.  A segment that crosses chunk boundaries leaves one partial sum per chunk
//       (slot A: the piece that began before the chunk, slot B: the piece that runs past it),
//       and K7b, launched over chunks, finishes each such segment from the chunk where it
//       starts by adding its partials in chunk order.  Every sum has a fixed order, so the
//       update is bitwise reproducible; no atomics.
#include "common.h"

namespace dlrm {

int check_csr_on_device(const int64_t *rows, int32_t T, const int64_t *indices,
                        const int64_t *offsets, int64_t B, int64_t nnz, int *flag,
                        hipStream_t stream);

namespace {

constexpr int kSortItems = 16;
constexpr int kSortTile = 256 * kSortItems;  // keys per sort / segment block

// ---------------------------------------------------------------- workspace layout

struct Layout {
    size_t keys_a, keys_b, vals_a, vals_b, bag_of, counts, totals, flag, seg_count, part_a, part_b,
        total;
    uint32_t nblk;    // sort / segment tiles
    uint32_t nchunk;  // K7 chunks
    int G, W;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool bwd_geometry(int32_t D, int *G, int *W) {
    if (D < 4 || D > 512 || (D & (D - 1)) != 0) return false;
    *G = D >= 64 ? 64 : D;
    *W = D / *G;
    return true;
}

Layout make_layout(int32_t D, int64_t nnz) {
    Layout L{};
    bwd_geometry(D, &L.G, &L.W);
    const size_t n = static_cast<size_t>(nnz > 0 ? nnz : 1);
    L.nblk = static_cast<uint32_t>((n + kSortTile - 1) / kSortTile);
    L.nchunk = static_cast<uint32_t>((n + L.G - 1) / L.G);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    L.keys_a = take(4 * n);
    L.keys_b = take(4 * n);
    L.vals_a = take(4 * n);
    L.vals_b = take(4 * n);
    L.bag_of = take(4 * n);
    L.counts = take(4 * 256 * static_cast<size_t>(L.nblk));
    L.totals = take(4 * 256);
    L.flag = take(4);
    L.seg_count = take(4 * static_cast<size_t>(L.nblk));
    L.part_a = take(4 * static_cast<size_t>(L.nchunk) * D);
    L.part_b = take(4 * static_cast<size_t>(L.nchunk) * D);
    L.total = off;
    return L;
}

// ---------------------------------------------------------------- scans

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive scan over a 256-thread block; every thread must call it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *total) {
    __shared__ uint32_t ws[4];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == 63) ws[w] = inc;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        off += (k < w) ? ws[k] : 0u;
        tot += ws[k];
    }
    __syncthreads();
    *total = tot;
    return off + inc - v;
}

// ---------------------------------------------------------------- K4 expand

struct ExpandArgs {
    uint32_t rowbase[kMaxTables];
    const int64_t *offsets;
    const int64_t *indices;
    uint32_t *keys;
    uint32_t *vals;
    uint32_t *bag_of;
    uint32_t B;
    uint32_t nbags;
};

__global__ __launch_bounds__(256) void k_expand(ExpandArgs a) {
    __shared__ int64_t so[257];
    const uint32_t g0 = blockIdx.x * 256u;
    const int nb = static_cast<int>(min(256u, a.nbags - g0));
    for (int i = threadIdx.x; i <= nb; i += 256) so[i] = a.offsets[g0 + i];
    __syncthreads();
    const int64_t p0 = so[0], p1 = so[nb];
    for (int64_t j = p0 + threadIdx.x; j < p1; j += 256) {
        int lo = 0, hi = nb;  // so[lo] <= j < so[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (so[mid] <= j) lo = mid;
            else hi = mid;
        }
        const uint32_t bag = g0 + lo;
        const uint32_t t = bag / a.B;
        a.keys[j] = a.rowbase[t] + static_cast<uint32_t>(a.indices[j]);
        a.vals[j] = static_cast<uint32_t>(j);
        a.bag_of[j] = bag;
    }
}

// ---------------------------------------------------------------- K5 radix sort

__global__ __launch_bounds__(256) void k_radix_hist(const uint32_t *__restrict__ keys, uint32_t n,
                                                    int shift, uint32_t *__restrict__ counts,
                                                    uint32_t nblk) {
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t base = blockIdx.x * kSortTile;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t k = base + i * 256 + threadIdx.x;
        if (k < n) atomicAdd(&h[(keys[k] >> shift) & 255u], 1u);
    }
    __syncthreads();
    counts[threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// Block d: exclusive scan of counts[d][0..nblk) in place; totals[d] = row sum.
__global__ __launch_bounds__(256) void k_radix_scan(uint32_t *__restrict__ counts, uint32_t nblk,
                                                    uint32_t *__restrict__ totals) {
    uint32_t *row = counts + static_cast<size_t>(blockIdx.x) * nblk;
    const uint32_t per = (nblk + 255) / 256;
    const uint32_t b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
    uint32_t s = 0;
    for (uint32_t i = b0; i < b1; ++i) s += row[i];
    uint32_t tot;
    uint32_t run = block_exclusive_scan(s, &tot);
    for (uint32_t i = b0; i < b1; ++i) {
        const uint32_t c = row[i];
        row[i] = run;
        run += c;
    }
    if (threadIdx.x == 0) totals[blockIdx.x] = tot;
}

__global__ __launch_bounds__(256) void k_radix_scatter(const uint32_t *__restrict__ kin,
                                                       const uint32_t *__restrict__ vin,
                                                       uint32_t *__restrict__ kout,
                                                       uint32_t *__restrict__ vout, uint32_t n,
                                                       int shift, const uint32_t *__restrict__ counts,
                                                       uint32_t nblk,
                                                       const uint32_t *__restrict__ totals) {
    __shared__ uint32_t dbase[256];
    __shared__ uint32_t wcnt[4][256];
    const int tid = threadIdx.x, w = tid >> 6;
    {
        uint32_t tot;
        const uint32_t excl = block_exclusive_scan(totals[tid], &tot);
        dbase[tid] = excl + counts[tid * nblk + blockIdx.x];
#pragma unroll
        for (int k = 0; k < 4; ++k) wcnt[k][tid] = 0;
    }
    __syncthreads();
    const uint32_t base = blockIdx.x * kSortTile + w * (kSortTile / 4) + (tid & 63);
    uint32_t key[kSortItems], val[kSortItems], loc[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t k = base + i * kWave;
        key[i] = k < n ? kin[k] : 0u;
        val[i] = k < n ? vin[k] : 0u;
    }
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const bool valid = base + i * kWave < n;
        const uint32_t d = (key[i] >> shift) & 255u;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (d >> bit) & 1u;
            const uint64_t m = __ballot(on);
            peers &= on ? m : ~m;
        }
        if (valid) {
            const uint32_t before = wcnt[w][d];
            loc[i] = before + __popcll(peers & lt);
            if ((peers & lt) == 0) wcnt[w][d] = before + __popcll(peers);
        }
    }
    __syncthreads();
    {
        const uint32_t c0 = wcnt[0][tid], c1 = wcnt[1][tid], c2 = wcnt[2][tid];
        const uint32_t b = dbase[tid];
        wcnt[0][tid] = b;
        wcnt[1][tid] = b + c0;
        wcnt[2][tid] = b + c0 + c1;
        wcnt[3][tid] = b + c0 + c1 + c2;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        if (base + i * kWave < n) {
            const uint32_t d = (key[i] >> shift) & 255u;
            const uint32_t pos = wcnt[w][d] + loc[i];
            kout[pos] = key[i];
            vout[pos] = val[i];
        }
    }
}

// ---------------------------------------------------------------- K6 unique + segments

__device__ __forceinline__ bool seg_flag(const uint32_t *keys, uint32_t k, uint32_t n) {
    return k < n && (k == 0 || keys[k] != keys[k - 1]);
}

__global__ __launch_bounds__(256) void k_seg_count(const uint32_t *__restrict__ keys, uint32_t n,
                                                   uint32_t *__restrict__ bcount) {
    uint32_t c = 0;
    const uint32_t base = blockIdx.x * kSortTile;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) c += seg_flag(keys, base + i * 256 + threadIdx.x, n);
    uint32_t tot;
    block_exclusive_scan(c, &tot);
    if (threadIdx.x == 0) bcount[blockIdx.x] = tot;
}

// One block: exclusive scan of the per-tile segment counts; U and the closing offset.
__global__ __launch_bounds__(256) void k_seg_scan(uint32_t *__restrict__ bcount, uint32_t nblk,
                                                  uint32_t n, int64_t *__restrict__ num_unique,
                                                  int64_t *__restrict__ seg_offsets) {
    const uint32_t per = (nblk + 255) / 256;
    const uint32_t b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
    uint32_t s = 0;
    for (uint32_t i = b0; i < b1; ++i) s += bcount[i];
    uint32_t tot;
    uint32_t run = block_exclusive_scan(s, &tot);
    for (uint32_t i = b0; i < b1; ++i) {
        const uint32_t c = bcount[i];
        bcount[i] = run;
        run += c;
    }
    if (threadIdx.x == 0) {
        if (num_unique) *num_unique = tot;
        if (seg_offsets) seg_offsets[tot] = n;
    }
}

__global__ __launch_bounds__(256) void k_seg_write(const uint32_t *__restrict__ keys, uint32_t n,
                                                   const uint32_t *__restrict__ bbase,
                                                   int64_t *__restrict__ unique_keys,
                                                   int64_t *__restrict__ seg_offsets) {
    __shared__ uint32_t wtot[4];
    const int tid = threadIdx.x, w = tid >> 6;
    const uint32_t base = blockIdx.x * kSortTile + w * (kSortTile / 4) + (tid & 63);
    uint64_t masks[kSortItems];
    uint32_t wsum = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        masks[i] = __ballot(seg_flag(keys, base + i * kWave, n));
        wsum += __popcll(masks[i]);
    }
    if ((tid & 63) == 0) wtot[w] = wsum;
    __syncthreads();
    uint32_t run = bbase[blockIdx.x];
    for (int k = 0; k < w; ++k) run += wtot[k];
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t k = base + i * kWave;
        if ((masks[i] >> (tid & 63)) & 1ull) {
            const uint32_t seg = run + __popcll(masks[i] & lt);
            if (unique_keys) unique_keys[seg] = keys[k];
            if (seg_offsets) seg_offsets[seg] = k;
        }
        run += __popcll(masks[i]);
    }
}

__global__ void k_empty_outputs(int64_t *num_unique, int64_t *seg_offsets) {
    if (num_unique) *num_unique = 0;
    if (seg_offsets) seg_offsets[0] = 0;
}

// ---------------------------------------------------------------- K7 segment reduce + Adagrad

struct AdagradArgs {
    char *tables[kMaxTables];
    float *state[kMaxTables];
    uint32_t rowbase[kMaxTables];
    const uint32_t *skeys;
    const uint32_t *perm;
    const uint32_t *bag_of;
    const float *weights;
    const float *grad;  // [B][T][D]
    float *part_a;
    float *part_b;
    uint32_t n;
    uint32_t nchunk;
    uint32_t B;
    int32_t T;
    int32_t D;
    float lr;
    float eps;
    float inv_D;
};

template <int DT, int W>
struct RowIO {
    // W consecutive elements of a table row, widened to fp32
    static __device__ __forceinline__ void load(const char *p, float *x) {
        if constexpr (DT == DLRM_F32) {
            const float *f = reinterpret_cast<const float *>(p);
            if constexpr (W == 1) x[0] = f[0];
            else if constexpr (W == 2) {
                const float2 v = *reinterpret_cast<const float2 *>(f);
                x[0] = v.x, x[1] = v.y;
            } else {
#pragma unroll
                for (int q = 0; q < W; q += 4) {
                    const float4 v = *reinterpret_cast<const float4 *>(f + q);
                    x[q] = v.x, x[q + 1] = v.y, x[q + 2] = v.z, x[q + 3] = v.w;
                }
            }
        } else {
            const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
            if constexpr (W == 1) x[0] = __uint_as_float(static_cast<uint32_t>(h[0]) << 16);
            else if constexpr (W == 2) {
                const uint32_t v = *reinterpret_cast<const uint32_t *>(h);
                x[0] = bf16_lo(v), x[1] = bf16_hi(v);
            } else if constexpr (W == 4) {
                const uint2 v = *reinterpret_cast<const uint2 *>(h);
                x[0] = bf16_lo(v.x), x[1] = bf16_hi(v.x), x[2] = bf16_lo(v.y), x[3] = bf16_hi(v.y);
            } else {
                const uint4 v = *reinterpret_cast<const uint4 *>(h);
                const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) x[2 * e] = bf16_lo(q[e]), x[2 * e + 1] = bf16_hi(q[e]);
            }
        }
    }
    static __device__ __forceinline__ void store(char *p, const float *x) {
        if constexpr (DT == DLRM_F32) {
            float *f = reinterpret_cast<float *>(p);
            if constexpr (W == 1) f[0] = x[0];
            else if constexpr (W == 2) *reinterpret_cast<float2 *>(f) = make_float2(x[0], x[1]);
            else {
#pragma unroll
                for (int q = 0; q < W; q += 4)
                    *reinterpret_cast<float4 *>(f + q) = make_float4(x[q], x[q + 1], x[q + 2], x[q + 3]);
            }
        } else {
            uint16_t *h = reinterpret_cast<uint16_t *>(p);
            uint32_t b[W];
#pragma unroll
            for (int e = 0; e < W; ++e) b[e] = f32_to_bf16_rne(x[e]);
            if constexpr (W == 1) h[0] = static_cast<uint16_t>(b[0]);
            else if constexpr (W == 2) *reinterpret_cast<uint32_t *>(h) = b[0] | (b[1] << 16);
            else if constexpr (W == 4)
                *reinterpret_cast<uint2 *>(h) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
            else
                *reinterpret_cast<uint4 *>(h) = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16),
                                                           b[4] | (b[5] << 16), b[6] | (b[7] << 16));
        }
    }
};

template <int W>
__device__ __forceinline__ void load_f32(const float *p, float *x) {
    RowIO<DLRM_F32, W>::load(reinterpret_cast<const char *>(p), x);
}
template <int W>
__device__ __forceinline__ void store_f32(float *p, const float *x) {
    RowIO<DLRM_F32, W>::store(reinterpret_cast<char *>(p), x);
}

// Sum of x over the G lanes of this lane group (butterfly: identical bits in every lane).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int s = 1; s < G; s <<= 1) x += __shfl_xor(x, s);
    return x;
}

// Row-wise Adagrad on one row: s += mean(G^2); row -= lr * G / (sqrt(s) + eps).
template <int DT, int W, int G>
__device__ __forceinline__ void adagrad_row(const AdagradArgs &a, uint32_t t, uint32_t r, int c,
                                            const float *g, const float *old_row, float old_state) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < W; ++e) ss = fmaf(g[e], g[e], ss);
    ss = group_sum<G>(ss);
    const float s_new = old_state + ss * a.inv_D;
    const float den = sqrtf(s_new) + a.eps;
    float nw[W];
#pragma unroll
    for (int e = 0; e < W; ++e) nw[e] = old_row[e] - a.lr * g[e] / den;
    constexpr int ES = DT == DLRM_BF16 ? 2 : 4;
    RowIO<DT, W>::store(a.tables[t] + (static_cast<uint64_t>(r) * a.D + c * W) * ES, nw);
    if (c == 0) a.state[t][r] = s_new;
}

template <int DT, int W, int G, bool WEIGHTED>
__global__ __launch_bounds__(256) void k_seg_reduce_adagrad(AdagradArgs a) {
    constexpr int NG = kWave / G;
    constexpr int U = 8;
    constexpr int ES = DT == DLRM_BF16 ? 2 : 4;
    const int lane = threadIdx.x & 63, grp = lane / G, c = lane % G, gbase = grp * G;
    const uint32_t chunk = (blockIdx.x * 4 + (threadIdx.x >> 6)) * NG + grp;
    if (chunk >= a.nchunk) return;  // group-uniform
    const uint32_t lo = chunk * G, hi = min(lo + G, a.n), cnt = hi - lo;

    // per-position metadata, one position per lane of the group
    const uint32_t k = lo + c;
    const bool have = k < hi;
    const uint32_t mykey = have ? a.skeys[k] : 0u;
    const uint32_t j = have ? a.perm[k] : 0u;
    const uint32_t mybag = have ? a.bag_of[j] : 0u;
    const float myw = (WEIGHTED && have) ? a.weights[j] : 1.f;
    const uint32_t key_lo = a.skeys[lo];
    bool open_before = lo > 0 && a.skeys[lo - 1] == key_lo;  // first piece began in an earlier chunk
    const bool runs_past = hi < a.n && a.skeys[hi] == a.skeys[hi - 1];

    float acc[W];
#pragma unroll
    for (int e = 0; e < W; ++e) acc[e] = 0.f;
    uint32_t cur = key_lo, cur_t = 0, cur_r = 0;
    float cur_row[W], cur_state = 0.f;
#pragma unroll
    for (int e = 0; e < W; ++e) cur_row[e] = 0.f;

    for (uint32_t r0 = 0; r0 < cnt; r0 += U) {
        float gr[U][W], tr[U][W], st[U], wu[U];
        uint32_t key[U], tt[U], rr[U];
        bool starts[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t r = r0 + u;
            const bool ok = r < cnt;
            const int src = gbase + (ok ? static_cast<int>(r) : 0);
            key[u] = __shfl(mykey, src);
            const uint32_t bag = __shfl(mybag, src);
            wu[u] = WEIGHTED ? __shfl(myw, src) : 1.f;
            // does position lo + r open a new segment?  (the first one may continue one)
            const uint32_t prev = __shfl(mykey, gbase + (r > 0 && ok ? static_cast<int>(r) - 1 : 0));
            starts[u] = ok && (r == 0 ? !open_before : key[u] != prev);
            tt[u] = bag / a.B;
            const uint32_t b = bag - tt[u] * a.B;
            rr[u] = key[u] - a.rowbase[tt[u]];
            if (ok) load_f32<W>(a.grad + (static_cast<uint64_t>(b) * a.T + tt[u]) * a.D + c * W, gr[u]);
            else {
#pragma unroll
                for (int e = 0; e < W; ++e) gr[u][e] = 0.f;
            }
            if (starts[u]) {
                RowIO<DT, W>::load(a.tables[tt[u]] + (static_cast<uint64_t>(rr[u]) * a.D + c * W) * ES,
                                   tr[u]);
                st[u] = a.state[tt[u]][rr[u]];
            } else {
#pragma unroll
                for (int e = 0; e < W; ++e) tr[u][e] = 0.f;
                st[u] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r0 + u >= cnt) break;
            if (starts[u]) {
                if (r0 + u > 0) {  // close the previous segment: it ended inside this chunk
                    if (open_before) store_f32<W>(a.part_a + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
                    else adagrad_row<DT, W, G>(a, cur_t, cur_r, c, acc, cur_row, cur_state);
                }
                open_before = false;
                cur = key[u];
                cur_t = tt[u];
                cur_r = rr[u];
#pragma unroll
                for (int e = 0; e < W; ++e) {
                    cur_row[e] = tr[u][e];
                    acc[e] = 0.f;
                }
                cur_state = st[u];
            }
#pragma unroll
            for (int e = 0; e < W; ++e) acc[e] = WEIGHTED ? fmaf(wu[u], gr[u][e], acc[e]) : acc[e] + gr[u][e];
        }
    }
    // the last piece of the chunk
    (void)cur;
    if (open_before) store_f32<W>(a.part_a + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
    else if (runs_past) store_f32<W>(a.part_b + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
    else adagrad_row<DT, W, G>(a, cur_t, cur_r, c, acc, cur_row, cur_state);
}

// Finishes the segments that cross chunk boundaries, each from the chunk where it starts.
template <int DT, int W, int G>
__global__ __launch_bounds__(256) void k_seg_finish(AdagradArgs a) {
    constexpr int NG = kWave / G;
    constexpr int ES = DT == DLRM_BF16 ? 2 : 4;
    constexpr int BATCH = 16;
    const int lane = threadIdx.x & 63, grp = lane / G, c = lane % G;
    const uint32_t chunk = (blockIdx.x * 4 + (threadIdx.x >> 6)) * NG + grp;
    if (chunk >= a.nchunk) return;
    const uint32_t lo = chunk * G, hi = min(lo + G, a.n);
    if (hi >= a.n) return;
    const uint32_t K = a.skeys[hi - 1];
    if (a.skeys[hi] != K) return;  // the last segment of this chunk ends here
    // does that segment start inside this chunk?
    if (a.skeys[lo] == K && lo > 0 && a.skeys[lo - 1] == K) return;
    // its piece in this chunk is in slot B (also when it starts exactly at lo)
    float acc[W];
    load_f32<W>(a.part_b + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
    // add slot A of the following chunks while the segment continues into them
    for (uint32_t c1 = chunk + 1;; c1 += BATCH) {
        bool in[BATCH];
        float pa[BATCH][W];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const uint64_t pos = static_cast<uint64_t>(c1 + i) * G;
            in[i] = pos < a.n && a.skeys[pos] == K;
            if (in[i]) load_f32<W>(a.part_a + static_cast<uint64_t>(c1 + i) * a.D + c * W, pa[i]);
        }
        bool more = true;
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if (!in[i]) {
                more = false;
                break;
            }
#pragma unroll
            for (int e = 0; e < W; ++e) acc[e] += pa[i][e];
        }
        if (!more) break;
    }
    // table and row of K
    const uint32_t bag = a.bag_of[a.perm[hi - 1]];
    const uint32_t t = bag / a.B;
    const uint32_t r = K - a.rowbase[t];
    float row[W];
    RowIO<DT, W>::load(a.tables[t] + (static_cast<uint64_t>(r) * a.D + c * W) * ES, row);
    adagrad_row<DT, W, G>(a, t, r, c, acc, row, a.state[t][r]);
}

template <int DT, int W, int G>
void launch_k7(const AdagradArgs &a, bool weighted, hipStream_t stream) {
    constexpr int NG = kWave / G;
    const uint32_t blocks = (a.nchunk + 4 * NG - 1) / (4 * NG);
    if (weighted)
        hipLaunchKernelGGL((k_seg_reduce_adagrad<DT, W, G, true>), dim3(blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((k_seg_reduce_adagrad<DT, W, G, false>), dim3(blocks), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((k_seg_finish<DT, W, G>), dim3(blocks), dim3(256), 0, stream, a);
}

template <int DT>
void dispatch_k7(const AdagradArgs &a, int G, int W, bool weighted, hipStream_t stream) {
    if (G == 64) {
        switch (W) {
            case 1: launch_k7<DT, 1, 64>(a, weighted, stream); break;
            case 2: launch_k7<DT, 2, 64>(a, weighted, stream); break;
            case 4: launch_k7<DT, 4, 64>(a, weighted, stream); break;
            case 8: launch_k7<DT, 8, 64>(a, weighted, stream); break;
        }
    } else {
        switch (G) {
            case 4: launch_k7<DT, 1, 4>(a, weighted, stream); break;
            case 8: launch_k7<DT, 1, 8>(a, weighted, stream); break;
            case 16: launch_k7<DT, 1, 16>(a, weighted, stream); break;
            case 32: launch_k7<DT, 1, 32>(a, weighted, stream); break;
        }
    }
}

}  // namespace
}  // namespace dlrm

extern "C" size_t emb_bag_bwd_workspace_size(int32_t T, const int64_t *rows, int32_t D, int64_t B,
                                             int64_t nnz) {
    using namespace dlrm;
    int G, W;
    if (T < 1 || T > kMaxTables || !rows || B < 0 || nnz < 0 || !bwd_geometry(D, &G, &W)) return 0;
    return make_layout(D, nnz).total;
}

extern "C" int emb_bag_bwd_adagrad(void *const *tables, float *const *state, const int64_t *rows,
                                   int32_t T, int32_t D, int32_t dtype, const int64_t *indices,
                                   const int64_t *offsets, const float *per_sample_weights,
                                   int64_t B, int64_t nnz, const float *grad_pooled, float lr,
                                   float eps, void *workspace, size_t workspace_bytes,
                                   int64_t *unique_keys_out, int64_t *segment_offsets_out,
                                   int32_t *sorted_pos_out, int64_t *num_unique_out,
                                   uint32_t flags, dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    int rc = check_batch(const_cast<const void *const *>(tables), rows, T, D, dtype, indices,
                         offsets, per_sample_weights, B, nnz);
    if (rc != DLRM_OK) return rc;
    if (flags & ~DLRM_FLAG_CHECK_INDICES) return DLRM_ERR_INVALID_ARG;
    int G, W;
    if (!bwd_geometry(D, &G, &W) || (dtype == DLRM_BF16 && D < 8)) return DLRM_ERR_UNSUPPORTED;
    if (!state) return DLRM_ERR_INVALID_ARG;
    uint64_t sumV = 0;
    for (int t = 0; t < T; ++t) {
        if (!state[t] || !aligned(state[t], 4)) return DLRM_ERR_INVALID_ARG;
        sumV += static_cast<uint64_t>(rows[t]);
    }
    if (sumV > (uint64_t(1) << 32)) return DLRM_ERR_UNSUPPORTED;
    if (nnz > 0 && (!grad_pooled || !aligned(grad_pooled, 16))) return DLRM_ERR_INVALID_ARG;
    if (B == 0 && nnz != 0) return DLRM_ERR_INVALID_ARG;
    const Layout L = make_layout(D, nnz);
    if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256)) return DLRM_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);

    if (flags & DLRM_FLAG_CHECK_INDICES) {
        rc = check_csr_on_device(rows, T, indices, offsets, B, nnz,
                                 reinterpret_cast<int *>(ws + L.flag), stream);
        if (rc != DLRM_OK) return rc;
    }
    const bool want_seg = unique_keys_out || segment_offsets_out || num_unique_out;
    if (nnz == 0) {
        if (want_seg)
            hipLaunchKernelGGL(k_empty_outputs, dim3(1), dim3(1), 0, stream, num_unique_out,
                               segment_offsets_out);
        return launch_status();
    }
    const uint32_t n = static_cast<uint32_t>(nnz);
    uint32_t *keys_a = reinterpret_cast<uint32_t *>(ws + L.keys_a);
    uint32_t *keys_b = reinterpret_cast<uint32_t *>(ws + L.keys_b);
    uint32_t *vals_a = reinterpret_cast<uint32_t *>(ws + L.vals_a);
    uint32_t *vals_b = reinterpret_cast<uint32_t *>(ws + L.vals_b);
    uint32_t *bag_of = reinterpret_cast<uint32_t *>(ws + L.bag_of);
    uint32_t *counts = reinterpret_cast<uint32_t *>(ws + L.counts);
    uint32_t *totals = reinterpret_cast<uint32_t *>(ws + L.totals);
    uint32_t *seg_count = reinterpret_cast<uint32_t *>(ws + L.seg_count);

    // K4
    ExpandArgs ea{};
    uint64_t acc_rows = 0;
    for (int t = 0; t < T; ++t) {
        ea.rowbase[t] = static_cast<uint32_t>(acc_rows);
        acc_rows += static_cast<uint64_t>(rows[t]);
    }
    ea.offsets = offsets;
    ea.indices = indices;
    ea.keys = keys_a;
    ea.vals = vals_a;
    ea.bag_of = bag_of;
    ea.B = static_cast<uint32_t>(B);
    ea.nbags = static_cast<uint32_t>(T * B);
    hipLaunchKernelGGL(k_expand, dim3((ea.nbags + 255) / 256), dim3(256), 0, stream, ea);

    // K5: passes over the significant bits of the largest key (sumV - 1)
    int bits = 0;
    while (bits < 32 && ((sumV - 1) >> bits) != 0) ++bits;
    const int passes = (bits + 7) / 8;
    uint32_t *kin = keys_a, *vin = vals_a, *kout = keys_b, *vout = vals_b;
    for (int p = 0; p < passes; ++p) {
        const bool last = p + 1 == passes;
        uint32_t *vdst = (last && sorted_pos_out) ? reinterpret_cast<uint32_t *>(sorted_pos_out) : vout;
        hipLaunchKernelGGL(k_radix_hist, dim3(L.nblk), dim3(256), 0, stream, kin, n, 8 * p, counts, L.nblk);
        hipLaunchKernelGGL(k_radix_scan, dim3(256), dim3(256), 0, stream, counts, L.nblk, totals);
        hipLaunchKernelGGL(k_radix_scatter, dim3(L.nblk), dim3(256), 0, stream, kin, vin, kout, vdst,
                           n, 8 * p, counts, L.nblk, totals);
        kin = kout;
        vin = vdst;
        kout = (kout == keys_b) ? keys_a : keys_b;
        vout = (vout == vals_b) ? vals_a : vals_b;
    }
    const uint32_t *skeys = kin;
    const uint32_t *perm = vin;
    if (passes == 0 && sorted_pos_out) {
        if (hipMemcpyAsync(sorted_pos_out, vals_a, sizeof(uint32_t) * n, hipMemcpyDeviceToDevice,
                           stream) != hipSuccess)
            return DLRM_ERR_HIP;
        perm = reinterpret_cast<const uint32_t *>(sorted_pos_out);
    }

    // K6
    if (want_seg) {
        hipLaunchKernelGGL(k_seg_count, dim3(L.nblk), dim3(256), 0, stream, skeys, n, seg_count);
        hipLaunchKernelGGL(k_seg_scan, dim3(1), dim3(256), 0, stream, seg_count, L.nblk, n,
                           num_unique_out, segment_offsets_out);
        if (unique_keys_out || segment_offsets_out)
            hipLaunchKernelGGL(k_seg_write, dim3(L.nblk), dim3(256), 0, stream, skeys, n, seg_count,
                               unique_keys_out, segment_offsets_out);
    }

    // K7
    AdagradArgs a{};
    for (int t = 0; t < T; ++t) {
        a.tables[t] = static_cast<char *>(tables[t]);
        a.state[t] = state[t];
        a.rowbase[t] = ea.rowbase[t];
    }
    a.skeys = skeys;
    a.perm = perm;
    a.bag_of = bag_of;
    a.weights = per_sample_weights;
    a.grad = grad_pooled;
    a.part_a = reinterpret_cast<float *>(ws + L.part_a);
    a.part_b = reinterpret_cast<float *>(ws + L.part_b);
    a.n = n;
    a.nchunk = L.nchunk;
    a.B = static_cast<uint32_t>(B);
    a.T = T;
    a.D = D;
    a.lr = lr;
    a.eps = eps;
    a.inv_D = 1.0f / static_cast<float>(D);
    const bool weighted = per_sample_weights != nullptr;
    if (dtype == DLRM_F32) dispatch_k7<DLRM_F32>(a, L.G, L.W, weighted, stream);
    else dispatch_k7<DLRM_BF16>(a, L.G, L.W, weighted, stream);
    return launch_status();
}
