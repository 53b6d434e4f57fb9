// Embedding backward with row-wise Adagrad, in place (robocikowo.com "DLRM": the training
// sentence of the paragraph "Forward pass" names SGD/Adagrad; the lookup is linear in the
// table, so a row's gradient is the weighted sum of the pooled gradients of the bags that
// looked it up).
//
// Pipeline (all on the caller's stream, no host synchronisation):
//   K4  expand: for lookup j of bag (t, b): key_j = rowbase[t] + idx_j, and the payloads
//       pos_j = j, grow_j = b*T + t (the row of grad_pooled it reads) and, when weighted,
//       w_j.  One block per 256 bags; bag offsets and bag rows staged in LDS.
//   K5  stable LSD radix sort of the keys carrying the payloads.  Keys of `bits` bits take
//       ceil(bits/10) passes of equal digits of max(8, ceil(bits/passes)) bits (25-bit keys:
//       3 passes of 9 bits).  Per pass: per-tile digit histograms, a per-digit scan across
//       tiles, and a scatter that ranks each key inside its tile with wavefront ballots
//       (stable: ties keep their order) and writes the tile out in runs of equal digits.
//   K6  unique keys and segment offsets (flag = key differs from its predecessor; a scan of
//       the flags), and for every K7 chunk the segment of its last position.  Always run: K7b
//       reads the segment ends; the caller's output buffers receive them when given.
//   K7  chunked segment reduction fused with the update.  The sorted sequence is cut into
//       chunks of CS positions, one per lane group of G = D/W lanes (W fp32 columns per lane);
//       a group walks its chunk in order with U gradient rows in flight, summing
//       w * grad_pooled rows.  A segment inside one chunk is finished on the spot: row-wise
//       Adagrad on the table row and state prefetched with the gradient rows.  A segment that
//       crosses chunk boundaries leaves one partial sum per chunk (slot A: the piece that began
//       in an earlier chunk, slot B: the piece that runs past the chunk) and its first chunk is
//       queued on a worklist; K7b takes each listed segment with a whole block, reads its end
//       from the segment offsets, adds the partials in chunk order and applies the update.
//       Every sum has a fixed order, so the update is bitwise reproducible; no float atomics.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace dlrm {

int check_csr_on_device(const int64_t *rows, int32_t T, const void *indices, const void *offsets,
                        int32_t index_type, int64_t B, int64_t nnz, int *flag, hipStream_t stream);

namespace {

constexpr int kSortItems = 16;
constexpr int kSortTile = 256 * kSortItems;  // keys per sort / segment block

#ifndef DLRM_K7_U
#define DLRM_K7_U 8  // gradient rows in flight per lane group
#endif


// floor(n / d) for n < 2^31 by multiply-high (Granlund & Montgomery 1994; Hacker's Delight 10-9).
struct FastDiv {
    uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((uint64_t(1) << s) < d) ++s;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
    return FastDiv{d, static_cast<uint32_t>(m), s};
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv &f) {
    return (__umulhi(n, f.m) + n) >> f.s;
}

// ---------------------------------------------------------------- workspace layout

struct Layout {
    size_t keys[2], pos[2], grow[2], wgt[2], counts, totals, flag, seg_count, seg_offsets,
        chunk_seg, fin_count, fin_list, part_a, part_b, total;
    uint32_t nblk;    // sort / segment tiles
    uint32_t nchunk;  // K7 chunks of CS sorted positions
    int G, W, CS;
    bool short_chunks;  // CS is the shorter of the two chunk lengths
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// lanes per row (G) and fp32 columns per lane (W) of the K7 kernels
// W columns per lane (16 bytes of fp32), D/W lanes per row, in a lane group of G lanes: D/W
// rounded up to a power of two, so that groups tile the 64-lane wavefront.  The G - D/W lanes past
// the row address its last W columns again (every load stays inside the row) and neither store
// nor add to the row's mean square.
bool bwd_geometry(int32_t D, int *G, int *W) {
    if (D < 4 || D > 512 || D % 4 != 0) return false;
    *W = D > 256 ? 8 : 4;
    if (D % *W != 0) return false;
    int g = 1;
    while (g < D / *W) g <<= 1;
    *G = g;
    return true;
}

// Sorted positions per K7 chunk: G lanes times MP positions per lane, at most 64.  A batch of
// fewer than kShortChunkMax lookups takes chunks of half that length where the lane group allows
// it (32 instead of 64 at D = 128): at full length its segment reduce would have fewer than about
// two blocks per CU, each walking a longer chain of dependent batches of loads.
constexpr int64_t kShortChunkMax = int64_t(1) << 18;

constexpr int chunk_mp(int G, bool shorter) {
    return G >= 64 ? 1 : G >= 16 ? (shorter ? 32 / G : 64 / G) : (shorter ? 2 : 4);
}

Layout make_layout(int32_t D, int64_t nnz) {
    Layout L{};
    bwd_geometry(D, &L.G, &L.W);
    L.short_chunks = nnz < kShortChunkMax;
    L.CS = L.G * chunk_mp(L.G, L.short_chunks);
    const size_t n = static_cast<size_t>(nnz > 0 ? nnz : 1);
    L.nblk = static_cast<uint32_t>((n + kSortTile - 1) / kSortTile);
    L.nchunk = static_cast<uint32_t>((n + L.CS - 1) / L.CS);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    for (int i = 0; i < 2; ++i) {
        L.keys[i] = take(4 * n);
        L.pos[i] = take(4 * n);
        L.grow[i] = take(4 * n);
        L.wgt[i] = take(4 * n);
    }
    L.counts = take(4 * 1024 * static_cast<size_t>(L.nblk));  // up to 10-bit digits
    L.totals = take(4 * 1024);
    L.flag = take(4);
    L.seg_count = take(4 * static_cast<size_t>(L.nblk));
    L.seg_offsets = take(8 * (n + 1));
    L.chunk_seg = take(4 * static_cast<size_t>(L.nchunk));
    L.fin_count = take(4);
    L.fin_list = take(4 * static_cast<size_t>(L.nchunk));
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
    const int w = static_cast<int>(wave_id()), lane = threadIdx.x & 63;
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

// A thread's contiguous range [b0, b1) of a count array: its sum, and the range rewritten as
// the exclusive prefix starting at `run`.  Counts are loaded KB at a time (clamped in bounds),
// so a range costs one round trip per KB entries rather than one per entry.
template <int KB>
__device__ __forceinline__ uint32_t range_sum(const uint32_t *row, uint32_t b0, uint32_t b1) {
    uint32_t s = 0;
    for (uint32_t i0 = b0; i0 < b1; i0 += KB) {
        uint32_t v[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) v[k] = row[min(i0 + k, b1 - 1)];
#pragma unroll
        for (int k = 0; k < KB; ++k) s += i0 + k < b1 ? v[k] : 0u;
    }
    return s;
}

template <int KB>
__device__ __forceinline__ void range_exclusive(uint32_t *row, uint32_t b0, uint32_t b1, uint32_t run) {
    for (uint32_t i0 = b0; i0 < b1; i0 += KB) {
        uint32_t v[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) v[k] = row[min(i0 + k, b1 - 1)];
#pragma unroll
        for (int k = 0; k < KB; ++k)
            if (i0 + k < b1) {
                row[i0 + k] = run;
                run += v[k];
            }
    }
}

// ---------------------------------------------------------------- K4 expand

struct ExpandArgs {
    uint32_t rowbase[kMaxTables];
    const void *offsets;  // int64 or int32 (the kernel's IT)
    const void *indices;
    const float *weights;
    uint32_t *keys;
    uint32_t *pos;   // NULL: the first radix pass makes the positions itself
    uint32_t *grow;
    uint32_t *wgt;   // NULL: the first radix pass reads the caller's weights itself
    uint32_t B;
    uint32_t T;
    uint32_t nbags;
};

template <typename IT>
__global__ __launch_bounds__(256) void k_expand(ExpandArgs a) {
    const IT *offsets = static_cast<const IT *>(a.offsets);
    const IT *indices = static_cast<const IT *>(a.indices);
    __shared__ int64_t so[257];
    __shared__ uint32_t s_grow[256], s_base[256];
    const uint32_t g0 = blockIdx.x * 256u;
    const int nb = static_cast<int>(min(256u, a.nbags - g0));
    for (int i = threadIdx.x; i <= nb; i += 256) so[i] = offsets[g0 + i];
    if (static_cast<int>(threadIdx.x) < nb) {
        const uint32_t bag = g0 + threadIdx.x;
        const uint32_t t = bag / a.B, b = bag - t * a.B;
        s_grow[threadIdx.x] = b * a.T + t;
        s_base[threadIdx.x] = a.rowbase[t];
    }
    __syncthreads();
    const int64_t p0 = so[0], p1 = so[nb];
    // EU lookups per thread and round: their indices are loaded together (clamped in bounds)
    // before the first is used, so a round costs one load round trip
    constexpr int EU = 8;
    for (int64_t j0 = p0 + threadIdx.x; j0 < p1; j0 += 256 * EU) {
        IT ix[EU];
#pragma unroll
        for (int u = 0; u < EU; ++u) ix[u] = indices[min(j0 + u * 256, p1 - 1)];
#pragma unroll
        for (int u = 0; u < EU; ++u) {
            const int64_t j = j0 + u * 256;
            if (j >= p1) break;
            int lo = 0, hi = nb;  // so[lo] <= j < so[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (so[mid] <= j) lo = mid;
                else hi = mid;
            }
            a.keys[j] = s_base[lo] + static_cast<uint32_t>(ix[u]);
            if (a.pos) a.pos[j] = static_cast<uint32_t>(j);
            a.grow[j] = s_grow[lo];
            if (a.wgt) a.wgt[j] = __float_as_uint(a.weights[j]);
        }
    }
}

// ---------------------------------------------------------------- K5 radix sort

// Lanes of the wavefront holding a valid item with the same RB-bit digit as this lane: one
// ballot per digit bit (the wave's match mask of equal digits).
template <int RB>
__device__ __forceinline__ uint64_t digit_peers(uint32_t d, bool valid) {
    const uint64_t v = __ballot(valid);
    uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const uint32_t nd = ~d;
#pragma unroll
    for (int bit = 0; bit < RB; ++bit) {
        const uint64_t m = __ballot((d >> bit) & 1u);
        // all ones where this lane's bit is clear (keep the lanes whose bit is clear too), else zero
        const uint32_t flip = static_cast<uint32_t>(static_cast<int32_t>(nd << (31 - bit)) >> 31);
        lo &= static_cast<uint32_t>(m) ^ flip;
        hi &= static_cast<uint32_t>(m >> 32) ^ flip;
    }
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Digits of RB bits (8..10): K = 2^RB / 256 digits per thread in the per-digit phases.
// Per-tile digit counts with LDS atomics.  Each thread counts kSortItems consecutive keys and adds
// each run of equal digits with one atomic: after the first pass the keys arrive ordered by the
// lower digits, so a tile holds long runs of one digit (hot rows, few tables per tile), and
// atomics to one LDS address serialize.  (Counting equal digits once per wavefront with the
// ballot match mask, as the scatter ranks them, was slower: 35 against 29 us per pass.)
template <int RB>
__global__ __launch_bounds__(256) void k_radix_hist(const uint32_t *__restrict__ keys, uint32_t n,
                                                    int shift, uint32_t *__restrict__ counts,
                                                    uint32_t nblk) {
    constexpr int NBK = 1 << RB;
    static_assert(kSortItems % 4 == 0, "keys are loaded 4 at a time");
    __shared__ uint32_t h[NBK];
    // the scatter's tile mapping: each XCD counts (and later scatters) one contiguous range of
    // tiles, so its count writes for a digit share lines in its own L2
    const uint32_t tile = xcd_contiguous(blockIdx.x, gridDim.x);
    if (tile >= nblk) return;  // block-uniform, before any barrier
    for (int d = threadIdx.x; d < NBK; d += 256) h[d] = 0;
    __syncthreads();
    const uint32_t tile0 = tile * kSortTile, base = tile0 + threadIdx.x * kSortItems;
    // all of a thread's keys are loaded before the first atomic: interleaved, the compiler waits
    // for each load in turn
    uint32_t key[kSortItems];
    if (tile0 + kSortTile <= n) {  // a whole tile: 16-byte loads (base is a multiple of 16 keys)
#pragma unroll
        for (int i = 0; i < kSortItems; i += 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(keys + base + i);
            key[i] = v.x, key[i + 1] = v.y, key[i + 2] = v.z, key[i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kSortItems; ++i) key[i] = keys[min(base + i, n - 1)];
    }
    uint32_t cur = (key[0] >> shift) & (NBK - 1), run = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t d = (key[i] >> shift) & (NBK - 1);
        if (d != cur) {
            if (run) atomicAdd(&h[cur], run);
            cur = d, run = 0;
        }
        run += base + i < n ? 1u : 0u;
    }
    if (run) atomicAdd(&h[cur], run);
    __syncthreads();
    for (int d = threadIdx.x; d < NBK; d += 256) counts[d * nblk + tile] = h[d];
}

// Block d: exclusive scan of counts[d][0..nblk) in place; totals[d] = row sum.  Thread i takes
// the consecutive entries [i*per, i*per + per); up to 16 of them stay in registers between the
// sum and the prefix (one round of loads), more are loaded again for the prefix.
__global__ __launch_bounds__(256) void k_radix_scan(uint32_t *__restrict__ counts, uint32_t nblk,
                                                    uint32_t *__restrict__ totals) {
    constexpr uint32_t KR = 16;
    uint32_t *row = counts + static_cast<size_t>(blockIdx.x) * nblk;
    const uint32_t per = (nblk + 255) / 256;
    const uint32_t b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
    uint32_t tot;
    if (per <= KR) {  // block-uniform
        uint32_t v[KR], sum = 0;
#pragma unroll
        for (uint32_t k = 0; k < KR; ++k) v[k] = row[min(b0 + k, nblk - 1)];  // clamped in bounds
#pragma unroll
        for (uint32_t k = 0; k < KR; ++k) sum += b0 + k < b1 ? v[k] : 0u;
        uint32_t run = block_exclusive_scan(sum, &tot);  // its barrier orders every load before any store
#pragma unroll
        for (uint32_t k = 0; k < KR; ++k)
            if (b0 + k < b1) {
                row[b0 + k] = run;
                run += v[k];
            }
    } else {
        const uint32_t run = block_exclusive_scan(range_sum<16>(row, b0, b1), &tot);
        range_exclusive<16>(row, b0, b1, run);
    }
    if (threadIdx.x == 0) totals[blockIdx.x] = tot;
}

struct SortIO {
    const uint32_t *kin;
    uint32_t *kout;
    // payload words in: grad row, then weight and position when present.  A NULL input is the
    // identity (each item's own index: the original positions, in the first pass).
    const uint32_t *pin[3];
    uint32_t *pout[3];
};

// Sorts of at most kInlineScanTiles tiles skip the scan launch: each scatter block adds up the raw
// per-tile counts of its digits itself (at most 16 per digit, loaded together), which costs less
// than a launch when the whole pass is a few microseconds.
constexpr uint32_t kInlineScanTiles = 16;

// NP payload words travel with each key.  Each 256-thread block ranks its tile of 4096 keys
// stably with wavefront ballots, stages the tile in LDS in sorted order, and writes it out in
// runs of equal digits, so the global stores are contiguous.  INL: counts are the raw per-tile
// counts (no scan ran; nblk <= kInlineScanTiles) and totals is unused.
template <int NP, int RB, bool INL>
__global__ __launch_bounds__(256) void k_radix_scatter(SortIO io, uint32_t n, int shift,
                                                       const uint32_t *__restrict__ counts,
                                                       uint32_t nblk,
                                                       const uint32_t *__restrict__ totals) {
    constexpr int NBK = 1 << RB;
    constexpr int K = NBK / 256;             // digits per thread in the per-digit phases
    constexpr uint32_t MASK = NBK - 1;
    __shared__ uint32_t gbase[NBK];  // global start of this block's run of digit d
    __shared__ uint32_t lbase[NBK];  // start of digit d inside the block's sorted tile
    __shared__ uint32_t wcnt[4][NBK];
    __shared__ uint32_t stage[kSortTile];
    // tiles are spread over the XCDs in contiguous ranges: the runs that neighbouring tiles write
    // for one digit are adjacent in the output, and meet in one L2 before they are written back
    const uint32_t tile = xcd_contiguous(blockIdx.x, gridDim.x);
    if (tile >= nblk) return;  // block-uniform, before any barrier
    const int tid = threadIdx.x, w = static_cast<int>(wave_id());
    // the tile's keys and payloads are loaded first: their round trip then overlaps the one of the
    // digit totals and counts below (in order, before the barriers the prologue needs)
    const uint32_t tile0 = tile * kSortTile;
    const uint32_t base = tile0 + w * (kSortTile / 4) + (tid & 63);
    uint32_t key[kSortItems], loc[kSortItems], pay[NP][kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t k = min(base + i * kWave, n - 1);  // unconditional loads
        key[i] = io.kin[k];
#pragma unroll
        for (int q = 0; q < NP; ++q) pay[q][i] = io.pin[q] ? io.pin[q][k] : k;
    }
    {
        // digits tid*K .. tid*K+K-1: global base = exclusive scan of totals + this block's prefix
        uint32_t tv[K], cv[K], sum = 0;
        if constexpr (INL) {
            // the digit's total and its count over the tiles before this one, from the raw counts
            uint32_t c[K][kInlineScanTiles];
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (uint32_t i = 0; i < kInlineScanTiles; ++i)
                    c[k][i] = counts[(tid * K + k) * nblk + min(i, nblk - 1)];  // clamped in bounds
#pragma unroll
            for (int k = 0; k < K; ++k) {
                tv[k] = 0, cv[k] = 0;
#pragma unroll
                for (uint32_t i = 0; i < kInlineScanTiles; ++i) {
                    const uint32_t x = i < nblk ? c[k][i] : 0u;
                    tv[k] += x;
                    cv[k] += i < tile ? x : 0u;
                }
                sum += tv[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                tv[k] = totals[tid * K + k];
                cv[k] = counts[(tid * K + k) * nblk + tile];
                sum += tv[k];
            }
        }
        uint32_t tot;
        uint32_t run = block_exclusive_scan(sum, &tot);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int d = tid * K + k;
            gbase[d] = run + cv[k];
            run += tv[k];
#pragma unroll
            for (int q = 0; q < 4; ++q) wcnt[q][d] = 0;
        }
    }
    __syncthreads();
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const bool valid = base + i * kWave < n;
        const uint32_t d = (key[i] >> shift) & MASK;
        const uint64_t peers = digit_peers<RB>(d, valid);
        if (valid) {
            const uint32_t before = wcnt[w][d];
            loc[i] = before + __popcll(peers & lt);
            if ((peers & lt) == 0) wcnt[w][d] = before + __popcll(peers);
        }
    }
    __syncthreads();
    {
        uint32_t c[K][4], sum = 0;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[k][q] = wcnt[q][tid * K + k];
                sum += c[k][q];
            }
        uint32_t tot;
        uint32_t run = block_exclusive_scan(sum, &tot);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int d = tid * K + k;
            lbase[d] = run;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wcnt[q][d] = run;
                run += c[k][q];
            }
        }
    }
    __syncthreads();
    const uint32_t nvalid = min(static_cast<uint32_t>(kSortTile), n - tile0);
    // keys: stage in sorted order, then write runs
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        if (base + i * kWave < n) {
            loc[i] += wcnt[w][(key[i] >> shift) & MASK];  // position in the sorted tile
            stage[loc[i]] = key[i];
        }
    }
    __syncthreads();
    uint32_t dst[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
        const uint32_t q = j * 256 + tid;
        const uint32_t k = stage[min(q, nvalid - 1)];
        const uint32_t d = (k >> shift) & MASK;
        dst[j] = gbase[d] + (q - lbase[d]);
        if (q < nvalid) io.kout[dst[j]] = k;
    }
    // payloads, one staged pass each
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSortItems; ++i)
            if (base + i * kWave < n) stage[loc[i]] = pay[p][i];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kSortItems; ++j) {
            const uint32_t q = j * 256 + tid;
            if (q < nvalid) io.pout[p][dst[j]] = stage[q];
        }
    }
}

// ---------------------------------------------------------------- K6 unique + segments

// Segment-start flags of the positions base + i*stride (i < kSortItems), with their keys.  All
// keys are loaded (unconditionally, clamped in bounds) before the first compare, so they make one
// round trip together.
__device__ __forceinline__ void seg_flags(const uint32_t *keys, uint32_t base, uint32_t stride, uint32_t n,
                                          bool *flag, uint32_t *kv) {
    uint32_t prev[kSortItems];
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t kk = min(base + i * stride, n - 1);
        kv[i] = keys[kk];
        prev[i] = keys[kk > 0 ? kk - 1 : 0];
    }
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t k = base + i * stride;
        flag[i] = k < n && (k == 0 || kv[i] != prev[i]);
    }
}

__global__ __launch_bounds__(256) void k_seg_count(const uint32_t *__restrict__ keys, uint32_t n,
                                                   uint32_t *__restrict__ bcount) {
    bool flag[kSortItems];
    uint32_t kv[kSortItems];
    seg_flags(keys, blockIdx.x * kSortTile + threadIdx.x, 256, n, flag, kv);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) c += flag[i] ? 1u : 0u;
    uint32_t tot;
    block_exclusive_scan(c, &tot);
    if (threadIdx.x == 0) bcount[blockIdx.x] = tot;
}

// Writes segment offsets (and unique keys when asked), and for every chunk of CS sorted
// positions the segment index of the chunk's last position.
// The tile's first segment index is the sum of the earlier tiles' counts, which each block adds
// up itself (at most a few thousand counts, read from L2); the last tile also writes U, the
// closing offset, and empties the finisher's worklist.
__global__ __launch_bounds__(256) void k_seg_write(const uint32_t *__restrict__ keys, uint32_t n,
                                                   const uint32_t *__restrict__ bcount, uint32_t nblk,
                                                   int64_t *__restrict__ unique_keys,
                                                   int64_t *__restrict__ seg_offsets,
                                                   uint32_t *__restrict__ chunk_seg, uint32_t CS,
                                                   int64_t *__restrict__ num_unique,
                                                   uint32_t *__restrict__ fin_count) {
    __shared__ uint32_t wtot[4];
    const int tid = threadIdx.x, w = static_cast<int>(wave_id()), lane = tid & 63;
    const uint32_t base = blockIdx.x * kSortTile + w * (kSortTile / 4) + lane;
    bool flags[kSortItems];
    uint32_t kv[kSortItems];
    seg_flags(keys, base, kWave, n, flags, kv);
    const uint32_t per = (blockIdx.x + 255) / 256;
    const uint32_t c0 = tid * per, c1 = min(blockIdx.x, c0 + per);
    uint32_t first;  // segments that start in earlier tiles
    block_exclusive_scan(range_sum<16>(bcount, c0, c1), &first);
    uint64_t masks[kSortItems];
    uint32_t wsum = 0;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        masks[i] = __ballot(flags[i]);
        wsum += __popcll(masks[i]);
    }
    if (lane == 0) wtot[w] = wsum;
    __syncthreads();
    uint32_t run = first;
    for (int k = 0; k < w; ++k) run += wtot[k];
    if (blockIdx.x + 1 == nblk && tid == 0) {
        const uint32_t total = first + wtot[0] + wtot[1] + wtot[2] + wtot[3];
        if (num_unique) *num_unique = total;
        seg_offsets[total] = n;
        *fin_count = 0;  // the finisher worklist of this call starts empty
    }
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t k = base + i * kWave;
        const bool flag = (masks[i] >> lane) & 1ull;
        const uint32_t seg_incl = run + __popcll(masks[i] & lt) + (flag ? 1u : 0u);  // flags in [0, k]
        if (flag) {
            if (unique_keys) unique_keys[seg_incl - 1] = kv[i];
            seg_offsets[seg_incl - 1] = k;
        }
        if (k < n && ((k + 1) % CS == 0 || k + 1 == n)) chunk_seg[k / CS] = seg_incl - 1;
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
    const uint32_t *skeys;        // sorted keys
    const uint32_t *sgrow;        // grad_pooled row of each sorted position
    const float *swgt;            // weight of each sorted position (weighted only)
    const float *grad;            // [B][T][D]
    const int64_t *seg_offsets;   // [U+1]
    const uint32_t *chunk_seg;    // [nchunk]: segment of the chunk's last position
    uint32_t *fin_count;          // number of chunks in fin_list
    uint32_t *fin_list;           // chunks where a chunk-crossing segment starts
    float *part_a;
    float *part_b;
    uint32_t n;
    uint32_t nchunk;
    int32_t T;
    int32_t D;
    FastDiv divT;
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

struct TableLDS {
    char *tab[kMaxTables];
    float *state[kMaxTables];
    uint32_t rowbase[kMaxTables];
};

__device__ __forceinline__ void stage_tables(const AdagradArgs &a, TableLDS &s) {
    if (static_cast<int>(threadIdx.x) < a.T) {
        s.tab[threadIdx.x] = a.tables[threadIdx.x];
        s.state[threadIdx.x] = a.state[threadIdx.x];
        s.rowbase[threadIdx.x] = a.rowbase[threadIdx.x];
    }
    __syncthreads();
}

template <int W>
__device__ __forceinline__ void load_f32(const float *p, float *x) {
    RowIO<DLRM_F32, W>::load(reinterpret_cast<const char *>(p), x);
}
template <int W>
__device__ __forceinline__ void store_f32(float *p, const float *x) {
    RowIO<DLRM_F32, W>::store(reinterpret_cast<char *>(p), x);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum of x over the G lanes of this lane group; every lane ends with the same bits (each step
// adds two partial sums that commute).  Within 16-lane rows the exchange is DPP (quad
// permutes, half-row and row mirrors); across rows it is a cross-lane permute.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (G >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (G >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror
    if constexpr (G >= 16) x += dpp_f32<0x140>(x); // row_mirror
#pragma unroll
    for (int s = 16; s < G; s <<= 1) x += __shfl_xor(x, s);
    return x;
}

// W table elements as 32-bit words: fp32 one per word, bf16 two per word.
template <int DT, int W>
struct TabWords {
    static constexpr int N = DT == DLRM_BF16 ? W / 2 : W;
    static __device__ __forceinline__ void to_f32(const uint32_t *w, float *x) {
        if constexpr (DT == DLRM_F32) {
#pragma unroll
            for (int e = 0; e < W; ++e) x[e] = __uint_as_float(w[e]);
        } else {
#pragma unroll
            for (int e = 0; e < W / 2; ++e) x[2 * e] = bf16_lo(w[e]), x[2 * e + 1] = bf16_hi(w[e]);
        }
    }
    static __device__ __forceinline__ void from_f32(const float *x, uint32_t *w) {
        if constexpr (DT == DLRM_F32) {
#pragma unroll
            for (int e = 0; e < W; ++e) w[e] = __float_as_uint(x[e]);
        } else {
#pragma unroll
            for (int e = 0; e < W / 2; ++e) {  // v_cvt_pk_bf16_f32: round to nearest even
                const __bf16 lo = static_cast<__bf16>(x[2 * e]), hi = static_cast<__bf16>(x[2 * e + 1]);
                w[e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                       (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
            }
        }
    }
};

// The update of one row (the lane's W columns).  Row-wise Adagrad: s += mean(G^2);
// row -= lr*G/(sqrt(s)+eps).  SGD: row -= lr*G (no state).  `row` points at the lane's first
// column of the row, `old` holds those columns as stored; a lane past the row (`col` false) takes
// no part.
template <int DT, int W, int G, int OPT>
__device__ __forceinline__ void update_row(const AdagradArgs &a, char *row, float *state, int cg, bool col,
                                           const float *g, const uint32_t *old, float old_state) {
    using TW = TabWords<DT, W>;
    if constexpr (OPT == DLRM_OPT_SGD) {
        float x[W];
        TW::to_f32(old, x);
#pragma unroll
        for (int e = 0; e < W; ++e) x[e] = fmaf(-a.lr, g[e], x[e]);
        uint32_t nw[TW::N];
        TW::from_f32(x, nw);
        if (col) gstore_words<TW::N>(row, nw);
        (void)state, (void)cg, (void)old_state;
        return;
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < W; ++e) ss = fmaf(g[e], g[e], ss);
    ss = group_sum<G>(col ? ss : 0.f);
    const float s_new = old_state + ss * a.inv_D;
    // hardware square root and reciprocal (about 1 ulp each)
    const float step = a.lr * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(s_new) + a.eps);
    float x[W];
    TW::to_f32(old, x);
#pragma unroll
    for (int e = 0; e < W; ++e) x[e] = fmaf(-step, g[e], x[e]);
    uint32_t nw[TW::N];
    TW::from_f32(x, nw);
    if (col) gstore_words<TW::N>(row, nw);
    if (cg == 0) *(DLRM_GLOBAL float *)state = s_new;
}

// Per sorted position, staged in LDS by the lane that owns it and read back as broadcasts.
struct PosMeta {
    const float *grad_row;  // grad_pooled row of the position
    char *tab_row;          // table row of the position's key (used where a segment starts)
    float *state;           // that row's accumulator (used where a segment starts)
    float w;
    float s_old;            // the accumulator's value before the update (Adagrad)
};

// Waves per SIMD asked of the compiler for K7: 5 for unweighted bf16 rows at D = 128, which then
// fits in 95 registers without spilling (97, and 4 waves, otherwise: 502 against 495 us on the
// multi-hot workload); the other shapes would spill under that limit, and keep the default.
constexpr int k7_min_waves(int DT, int W, int G, bool weighted) {
    return DT == DLRM_BF16 && W == 4 && G == 32 && !weighted ? 5 : 1;
}

// Chunk of CS = G*MP sorted positions per lane group of G lanes; U gradient rows in flight.
template <int DT, int W, int G, int MP, bool WEIGHTED, int U, int OPT>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(k7_min_waves(DT, W, G, WEIGHTED)))) void k_seg_reduce_adagrad(AdagradArgs a) {
    using TW = TabWords<DT, W>;
    constexpr int NG = kWave / G;
    constexpr int CS = G * MP;
    constexpr int ES = DT == DLRM_BF16 ? 2 : 4;
    static_assert(CS <= 64, "start flags live in one 64-bit mask");
    __shared__ PosMeta meta[4][NG][CS];
    __shared__ TableLDS sl;
    stage_tables(a, sl);
    const int wv = static_cast<int>(wave_id()), lane = threadIdx.x & 63, grp = lane / G, cg = lane % G;
    const int dw = a.D / W;           // lanes that hold columns of the row
    const bool col = cg < dw;
    const int c = col ? cg : dw - 1;  // the lane's columns (past the row: the last W again)
    const uint32_t chunk = (blockIdx.x * 4 + wv) * NG + grp;
    if (chunk >= a.nchunk) return;  // group-uniform
    const uint32_t lo = chunk * CS, hi = min(lo + CS, a.n), cnt = hi - lo;
    PosMeta *pm = meta[wv][grp];
    // Keys that place the chunk's first and last segments against the neighbouring chunks, read
    // now (unconditionally, clamped in bounds) and used later: the key just before the previous
    // chunk, the chunk's first and last keys, the next position's key and the next chunk's last.
    const uint32_t e_next = min(hi + CS, a.n);  // end of the next chunk
    const uint32_t key_pp = a.skeys[chunk >= 2 ? lo - CS - 1 : 0];
    const uint32_t key_lo = a.skeys[lo];
    const uint32_t key_last = a.skeys[hi - 1];
    const uint32_t key_hi = a.skeys[min(hi, a.n - 1)];
    const uint32_t key_e = a.skeys[e_next - 1];

    // build the chunk's metadata: lane cg of the group owns positions lo + cg + m*G (every lane of
    // the group, also those past the row: ownership of positions does not depend on the columns)
    uint64_t starts = 0;  // bit r: position lo + r opens a segment
#pragma unroll
    for (int m = 0; m < MP; ++m) {
        const uint32_t r = cg + m * G, k = lo + r;
        const bool have = k < hi;
        const uint32_t kk = have ? k : hi - 1;  // loads stay unconditional
        const uint32_t key = a.skeys[kk];
        const uint32_t prev = a.skeys[kk > 0 ? kk - 1 : 0];
        const uint32_t grow = a.sgrow[kk];
        const float w = WEIGHTED ? a.swgt[kk] : 1.f;
        const bool st = have && (kk == 0 || key != prev);
        const uint32_t t = grow - fast_div(grow, a.divT) * a.divT.d;
        const uint32_t row = key - sl.rowbase[t];
        PosMeta p;
        p.grad_row = a.grad + static_cast<uint64_t>(grow) * a.D;
        p.tab_row = sl.tab[t] + static_cast<uint64_t>(row) * a.D * ES;
        p.state = OPT == DLRM_OPT_ADAGRAD ? sl.state[t] + row : nullptr;
        p.w = w;
        // read here, one lane per position, rather than by the whole group in the main loop (the
        // owning group is the only writer of this row's state, and it writes after this read)
        p.s_old = OPT == DLRM_OPT_ADAGRAD ? *(const DLRM_GLOBAL float *)p.state : 0.f;
        if (have) pm[r] = p;
        const uint64_t bal = __ballot(st);
        starts |= ((bal >> (grp * G)) & (G == 64 ? ~0ull : ((1ull << G) - 1))) << (m * G);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if (starts == 0) {
        // no segment starts here: the whole chunk continues one that began earlier, so it is
        // streamed straight into slot A with no per-position bookkeeping
        float acc[W];
#pragma unroll
        for (int e = 0; e < W; ++e) acc[e] = 0.f;
        for (uint32_t r0 = 0; r0 < cnt; r0 += U) {
            uint32_t gr[U][W];
            float wu[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const PosMeta &p = pm[min(r0 + u, cnt - 1)];
                gload_words<W>(p.grad_row + c * W, gr[u]);
                wu[u] = p.w;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (r0 + u < cnt) {
#pragma unroll
                    for (int e = 0; e < W; ++e) {
                        const float g = __uint_as_float(gr[u][e]);
                        acc[e] = WEIGHTED ? fmaf(wu[u], g, acc[e]) : acc[e] + g;
                    }
                }
            }
        }
        if (col) store_f32<W>(a.part_a + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
        return;
    }
    bool open_before = !(starts & 1ull);  // the first piece began in an earlier chunk
    const bool runs_past = hi < a.n && key_hi == key_last;
    // A segment that begins in one chunk and ends inside the next (before that chunk's last
    // position) belongs wholly to the chunk where it begins: that group reads on into the next
    // chunk and updates the row; the next chunk's group skips the segment's head.  Only longer
    // segments are cut into per-chunk partials for the finisher.  Keys are sorted, so the open
    // segment began inside the previous chunk iff the position before that chunk holds another
    // key, and the last segment ends inside the next chunk iff that chunk's last key differs.
    uint32_t r_begin = 0;
    if (open_before && (chunk < 2 || key_pp != key_lo)) {  // the previous chunk finishes it
        r_begin = static_cast<uint32_t>(__builtin_ctzll(starts));
        open_before = false;
    }

    float acc[W];
#pragma unroll
    for (int e = 0; e < W; ++e) acc[e] = 0.f;
    // the open segment: where it starts in the chunk (its table row and state pointers are
    // read back from the chunk's metadata when it is flushed), and its row and state as loaded
    uint32_t cur_r = 0;
    uint32_t cur_row[TW::N];
    float cur_s = 0.f;
#pragma unroll
    for (int e = 0; e < TW::N; ++e) cur_row[e] = 0u;
    auto flush = [&](uint32_t rs) {
        const PosMeta &p = pm[rs];
        update_row<DT, W, G, OPT>(a, p.tab_row + c * W * ES, p.state, cg, col, acc, cur_row, cur_s);
    };

    for (uint32_t r0 = 0; r0 < cnt; r0 += U) {
        // Every load below is unconditional (positions outside [r_begin, cnt) re-read a position
        // inside it), and every loaded value is consumed by a select rather than under a branch,
        // so the compiler neither sinks a load into a branch nor splits the batch: all of them
        // are in flight together, issued in the order they are used.
        uint32_t gr[U][W], tr[U][TW::N];
        float st[U], wu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const PosMeta &p = pm[min(max(r0 + u, r_begin), cnt - 1)];
            gload_words<W>(p.grad_row + c * W, gr[u]);
            // the table row of the position's key: used where a segment starts, and loaded at
            // every position (the row of the segment already being read: a cache hit)
            gload_words<TW::N>(p.tab_row + c * W * ES, tr[u]);
            st[u] = p.s_old;
            wu[u] = WEIGHTED ? p.w : 1.f;
            __builtin_amdgcn_sched_barrier(0);  // issue in use order: position u's loads arrive first
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t r = r0 + u;
            const bool valid = r < cnt && r >= r_begin;
            const bool s_u = valid && ((starts >> (r & 63u)) & 1ull);
            if (s_u) {
                if (r > r_begin) {  // the previous piece ended inside this chunk
                    if (open_before) {
                        if (col) store_f32<W>(a.part_a + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
                    }
                    else flush(cur_r);
                }
#pragma unroll
                for (int e = 0; e < W; ++e) acc[e] = 0.f;
            }
            open_before = open_before && !s_u;
            cur_r = s_u ? r : cur_r;
            cur_s = s_u ? st[u] : cur_s;
#pragma unroll
            for (int e = 0; e < TW::N; ++e) cur_row[e] = s_u ? tr[u][e] : cur_row[e];
#pragma unroll
            for (int e = 0; e < W; ++e) {
                const float g = valid ? __uint_as_float(gr[u][e]) : 0.f;
                acc[e] = WEIGHTED ? fmaf(valid ? wu[u] : 0.f, g, acc[e]) : acc[e] + g;
            }
        }
    }
    // the last piece of the chunk
    const bool carry_on = runs_past && key_e != key_last;
    if (open_before) {
        if (col) store_f32<W>(a.part_a + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
    } else if (carry_on) {
        // read on to the segment's end in the next chunk (fewer than CS positions), then update
        const uint32_t span = e_next - hi;  // positions of the next chunk
        char *row_ptr = pm[cur_r].tab_row + c * W * ES;
        float *st_ptr = pm[cur_r].state;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // every lane is done with this chunk's metadata
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint32_t m = 0;  // positions of the segment in the next chunk: its keys equal key_last
#pragma unroll
        for (int k = 0; k < MP; ++k) {
            const uint32_t r = cg + k * G;
            const uint32_t kk = hi + min(r, span - 1);
            const bool same = r < span && a.skeys[kk] == key_last;
            PosMeta p;
            p.grad_row = a.grad + static_cast<uint64_t>(a.sgrow[kk]) * a.D;
            p.tab_row = nullptr;
            p.state = nullptr;
            p.w = WEIGHTED ? a.swgt[kk] : 1.f;
            p.s_old = 0.f;
            if (same) pm[r] = p;
            const uint64_t bal = __ballot(same);
            m += static_cast<uint32_t>(__popcll((bal >> (grp * G)) & (G == 64 ? ~0ull : ((1ull << G) - 1))));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (uint32_t r0 = 0; r0 < m; r0 += U) {
            uint32_t gr[U][W];
            float wu[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const PosMeta &p = pm[min(r0 + u, m - 1)];
                gload_words<W>(p.grad_row + c * W, gr[u]);
                wu[u] = p.w;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (r0 + u < m) {
#pragma unroll
                    for (int e = 0; e < W; ++e) {
                        const float g = __uint_as_float(gr[u][e]);
                        acc[e] = WEIGHTED ? fmaf(wu[u], g, acc[e]) : acc[e] + g;
                    }
                }
            }
        }
        update_row<DT, W, G, OPT>(a, row_ptr, st_ptr, cg, col, acc, cur_row, cur_s);
    } else if (runs_past) {
        if (col) store_f32<W>(a.part_b + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
        // the segment starting here crosses into later chunks: queue it for the finisher
        // (list order is arbitrary; each entry's work is fixed, so results do not depend on it)
        if (cg == 0) a.fin_list[atomicAdd(a.fin_count, 1u)] = chunk;
    } else {
        flush(cur_r);
    }
}

// Finishes the chunk-crossing segments: a grid-stride loop over the worklist K7 filled, one
// listed chunk per block at a time.  The segment's partials are added in chunk order (slot B of
// its first chunk, then slot A of every later chunk it covers), then the row is updated.
// The first wavefront loads the chunk, the last chunk and the table row of up to 64 of the
// block's items at once, so an item waits on one round trip (its partials, row and state) rather
// than on the chain worklist -> segment -> segment end -> key -> row.
template <int DT, int W, int G, int CS, int OPT>
__global__ __launch_bounds__(256) void k_seg_finish(AdagradArgs a) {
    constexpr int NS = 256 / G;  // partial rows read per pass of the block
    constexpr int U = 8;
    constexpr int ES = DT == DLRM_BF16 ? 2 : 4;
    __shared__ float red[NS][G * W];
    __shared__ uint32_t s_chunk[kWave], s_ce[kWave], s_t[kWave], s_r[kWave];
    __shared__ TableLDS sl;
    stage_tables(a, sl);
    const int sub = threadIdx.x / G, cg = threadIdx.x % G;
    const int dw = a.D / W;           // lanes that hold columns of the row
    const bool col = cg < dw;
    const int c = col ? cg : dw - 1;  // the lane's columns (past the row: the last W again)
    const uint32_t count = *a.fin_count;
    for (uint32_t first = blockIdx.x; first < count; first += gridDim.x * kWave) {  // block-uniform
        if (threadIdx.x < kWave) {
            const uint32_t item = first + threadIdx.x * gridDim.x;
            const uint32_t chunk = a.fin_list[item < count ? item : first];
            const uint32_t u = a.chunk_seg[chunk];
            const uint32_t hi = chunk * CS + CS;
            const uint32_t K = a.skeys[hi - 1];
            const uint32_t grow = a.sgrow[hi - 1];
            const uint32_t t = grow - fast_div(grow, a.divT) * a.divT.d;
            s_chunk[threadIdx.x] = chunk;
            s_ce[threadIdx.x] = static_cast<uint32_t>((a.seg_offsets[u + 1] - 1) / CS);  // last chunk it covers
            s_t[threadIdx.x] = t;
            s_r[threadIdx.x] = K - sl.rowbase[t];
        }
        __syncthreads();
        for (uint32_t k = 0; k < kWave && first + k * gridDim.x < count; ++k) {  // block-uniform
            const uint32_t chunk = s_chunk[k], ce = s_ce[k], t = s_t[k], r = s_r[k];
            // the row and its state, loaded with the partials
            char *row = sl.tab[t] + (static_cast<uint64_t>(r) * a.D + c * W) * ES;
            float *st = OPT == DLRM_OPT_ADAGRAD ? sl.state[t] + r : nullptr;
            uint32_t old[TabWords<DT, W>::N];
            float s_old = 0.f;
            if (sub == 0) {
                gload_words<TabWords<DT, W>::N>(row, old);
                if constexpr (OPT == DLRM_OPT_ADAGRAD) s_old = *(const DLRM_GLOBAL float *)st;
            }
            float acc[W];
#pragma unroll
            for (int q = 0; q < W; ++q) acc[q] = 0.f;
            if (sub == 0) load_f32<W>(a.part_b + static_cast<uint64_t>(chunk) * a.D + c * W, acc);
            for (uint32_t c1 = chunk + 1 + sub; c1 <= ce; c1 += NS * U) {
                uint32_t pa[U][W];
#pragma unroll
                for (int kk = 0; kk < U; ++kk)  // unconditional loads (clamped), all in flight together
                    gload_words<W>(a.part_a + static_cast<uint64_t>(min(c1 + kk * NS, ce)) * a.D + c * W, pa[kk]);
#pragma unroll
                for (int kk = 0; kk < U; ++kk)
                    if (c1 + kk * NS <= ce)
#pragma unroll
                        for (int q = 0; q < W; ++q) acc[q] += __uint_as_float(pa[kk][q]);
            }
            // combine the NS row slots in a fixed order
#pragma unroll
            for (int q = 0; q < W; ++q) red[sub][cg * W + q] = acc[q];
            __syncthreads();
            if (sub == 0) {
#pragma unroll
                for (int q = 0; q < W; ++q) {
                    float x = red[0][cg * W + q];
                    for (int kk = 1; kk < NS; ++kk) x += red[kk][cg * W + q];
                    acc[q] = x;
                }
                update_row<DT, W, G, OPT>(a, row, st, cg, col, acc, old, s_old);
            }
            __syncthreads();  // red[] is reused by the next item
        }
        __syncthreads();  // the staged items are reused by the next batch
    }
}

template <int DT, int W, int G, int MP, int OPT>
void launch_k7_mp(const AdagradArgs &a, bool weighted, hipStream_t stream) {
    constexpr const char *name = OPT == DLRM_OPT_SGD ? "seg_reduce_sgd" : "seg_reduce_adagrad";
    constexpr int NG = kWave / G;
    constexpr int U = DLRM_K7_U;
    const uint32_t blocks = (a.nchunk + 4 * NG - 1) / (4 * NG);
    if (weighted)
        DLRM_LAUNCH(name, (k_seg_reduce_adagrad<DT, W, G, MP, true, U, OPT>), dim3(blocks), dim3(256), 0, stream, a);
    else
        DLRM_LAUNCH(name, (k_seg_reduce_adagrad<DT, W, G, MP, false, U, OPT>), dim3(blocks), dim3(256), 0, stream, a);
    const uint32_t fin_blocks = a.nchunk < 2048 ? a.nchunk : 2048;
    DLRM_LAUNCH("seg_finish", (k_seg_finish<DT, W, G, G * MP, OPT>), dim3(fin_blocks), dim3(256), 0, stream, a);
}

template <int DT, int W, int G, int OPT>
void launch_k7(const AdagradArgs &a, bool weighted, bool shorter, hipStream_t stream) {
    if (shorter) launch_k7_mp<DT, W, G, chunk_mp(G, true), OPT>(a, weighted, stream);
    else launch_k7_mp<DT, W, G, chunk_mp(G, false), OPT>(a, weighted, stream);
}

template <int DT, int OPT>
void dispatch_k7(const AdagradArgs &a, int G, int W, bool weighted, bool shorter, hipStream_t stream) {
    if (W == 8) {
        launch_k7<DT, 8, 64, OPT>(a, weighted, shorter, stream);
        return;
    }
    switch (G) {
        case 1: launch_k7<DT, 4, 1, OPT>(a, weighted, shorter, stream); break;
        case 2: launch_k7<DT, 4, 2, OPT>(a, weighted, shorter, stream); break;
        case 4: launch_k7<DT, 4, 4, OPT>(a, weighted, shorter, stream); break;
        case 8: launch_k7<DT, 4, 8, OPT>(a, weighted, shorter, stream); break;
        case 16: launch_k7<DT, 4, 16, OPT>(a, weighted, shorter, stream); break;
        case 32: launch_k7<DT, 4, 32, OPT>(a, weighted, shorter, stream); break;
        case 64: launch_k7<DT, 4, 64, OPT>(a, weighted, shorter, stream); break;
    }
}

template <int RB>
void launch_radix_pass(const SortIO &io, int NP, uint32_t n, int shift, uint32_t *counts,
                       uint32_t nblk, uint32_t *totals, hipStream_t stream) {
    DLRM_LAUNCH("radix_hist", k_radix_hist<RB>, dim3(round_up_xcd(nblk)), dim3(256), 0, stream, io.kin, n, shift,
                counts, nblk);
    const dim3 sgrid(round_up_xcd(nblk));
    if (nblk <= kInlineScanTiles) {
        if (NP == 3)
            DLRM_LAUNCH("radix_scatter", (k_radix_scatter<3, RB, true>), sgrid, dim3(256), 0, stream, io, n, shift,
                        counts, nblk, totals);
        else if (NP == 2)
            DLRM_LAUNCH("radix_scatter", (k_radix_scatter<2, RB, true>), sgrid, dim3(256), 0, stream, io, n, shift,
                        counts, nblk, totals);
        else
            DLRM_LAUNCH("radix_scatter", (k_radix_scatter<1, RB, true>), sgrid, dim3(256), 0, stream, io, n, shift,
                        counts, nblk, totals);
        return;
    }
    DLRM_LAUNCH("radix_scan", k_radix_scan, dim3(1 << RB), dim3(256), 0, stream, counts, nblk, totals);
    if (NP == 3)
        DLRM_LAUNCH("radix_scatter", (k_radix_scatter<3, RB, false>), sgrid, dim3(256), 0, stream, io, n, shift,
                    counts, nblk, totals);
    else if (NP == 2)
        DLRM_LAUNCH("radix_scatter", (k_radix_scatter<2, RB, false>), sgrid, dim3(256), 0, stream, io, n, shift,
                    counts, nblk, totals);
    else
        DLRM_LAUNCH("radix_scatter", (k_radix_scatter<1, RB, false>), sgrid, dim3(256), 0, stream, io, n, shift,
                    counts, nblk, totals);
}

}  // namespace
}  // namespace dlrm

extern "C" size_t emb_bag_bwd_workspace_size(int32_t T, const int64_t *rows, int32_t D, int64_t B,
                                             int64_t nnz) {
    using namespace dlrm;
    int G, W;
    if (T < 1 || T > kMaxTables || !rows || B < 0 || nnz < 0 || !bwd_geometry(D, &G, &W)) return 0;
    // a smaller batch may take the shorter chunks and then needs more partial rows: the size for
    // nnz lookups covers every batch of at most nnz
    size_t total = make_layout(D, nnz).total;
    if (nnz >= kShortChunkMax) total = std::max(total, make_layout(D, kShortChunkMax - 1).total);
    return total;
}

namespace dlrm {
namespace {

__global__ void k_zero_u32(uint32_t *p) { *p = 0; }

// What a plan leaves in the workspace and where: fixed by (rows, D, nnz, weighted).
struct PlanShape {
    Layout L;
    uint64_t sumV;
    int passes;
    int rb[4];  // digit width of each pass (8..10 bits)
    int cur;  // ping-pong half holding the sorted keys and payloads
};

int plan_shape(const int64_t *rows, int32_t T, int32_t D, int64_t nnz, PlanShape *ps) {
    uint64_t sumV = 0;
    for (int t = 0; t < T; ++t) sumV += static_cast<uint64_t>(rows[t]);
    if (sumV > (uint64_t(1) << 32)) return DLRM_ERR_UNSUPPORTED;
    ps->L = make_layout(D, nnz);
    ps->sumV = sumV;
    // passes over the significant bits of the largest key (sumV - 1), digits of 8..10 bits chosen
    // for the fewest passes
    int bits = 0;
    while (bits < 32 && ((sumV - 1) >> bits) != 0) ++bits;
    ps->passes = (bits + 9) / 10;
    // the bits split as evenly as they go, wider digits first, none narrower than 8 bits
    for (int p = 0; p < 4; ++p) {
        const int w = ps->passes > 0 ? bits / ps->passes + (p < bits % ps->passes ? 1 : 0) : 8;
        ps->rb[p] = w < 8 ? 8 : w;
    }
    ps->cur = ps->passes & 1;
    return DLRM_OK;
}

int check_rows(const int64_t *rows, int32_t T) {
    if (T < 1 || T > kMaxTables || !rows) return DLRM_ERR_INVALID_ARG;
    for (int t = 0; t < T; ++t)
        if (rows[t] < 1) return DLRM_ERR_INVALID_ARG;
    return DLRM_OK;
}

}  // namespace
}  // namespace dlrm

extern "C" int emb_bag_bwd_plan(const int64_t *rows, int32_t T, int32_t D, const void *indices,
                                const void *offsets, int32_t index_type, const float *per_sample_weights,
                                int64_t B, int64_t nnz, void *workspace, size_t workspace_bytes,
                                int64_t *unique_keys_out, int64_t *segment_offsets_out, int32_t *sorted_pos_out,
                                int64_t *num_unique_out, uint32_t flags, dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (index_type != DLRM_INDEX_I64 && index_type != DLRM_INDEX_I32) return DLRM_ERR_INVALID_ARG;
    int rc = check_rows(rows, T);
    if (rc != DLRM_OK) return rc;
    // the batch checks of the forward, with placeholder (never read) table pointers
    const void *fake_tables[kMaxTables];
    for (int t = 0; t < T; ++t) fake_tables[t] = reinterpret_cast<const void *>(uintptr_t(256));
    rc = check_batch(fake_tables, rows, T, D, DLRM_F32, indices, offsets, index_type, per_sample_weights, B, nnz);
    if (rc != DLRM_OK) return rc;
    if (flags & ~DLRM_FLAG_CHECK_INDICES) return DLRM_ERR_INVALID_ARG;
    int G, W;
    if (!bwd_geometry(D, &G, &W)) return DLRM_ERR_UNSUPPORTED;
    if (B == 0 && nnz != 0) return DLRM_ERR_INVALID_ARG;
    PlanShape ps;
    rc = plan_shape(rows, T, D, nnz, &ps);
    if (rc != DLRM_OK) return rc;
    const Layout &L = ps.L;
    if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256)) return DLRM_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    auto u32 = [&](size_t off) { return reinterpret_cast<uint32_t *>(ws + off); };

    if (flags & DLRM_FLAG_CHECK_INDICES) {
        rc = check_csr_on_device(rows, T, indices, offsets, index_type, B, nnz, reinterpret_cast<int *>(ws + L.flag),
                                 stream);
        if (rc != DLRM_OK) return rc;
    }
    if (nnz == 0) {
        if (unique_keys_out || segment_offsets_out || num_unique_out)
            DLRM_LAUNCH("empty_outputs", k_empty_outputs, dim3(1), dim3(1), 0, stream, num_unique_out,
                        segment_offsets_out);
        return launch_status();
    }
    const uint32_t n = static_cast<uint32_t>(nnz);
    const bool weighted = per_sample_weights != nullptr;

    // K4
    ExpandArgs ea{};
    uint64_t acc_rows = 0;
    for (int t = 0; t < T; ++t) {
        ea.rowbase[t] = static_cast<uint32_t>(acc_rows);
        acc_rows += static_cast<uint64_t>(rows[t]);
    }
    ea.offsets = offsets;
    ea.indices = indices;
    ea.weights = per_sample_weights;
    ea.keys = u32(L.keys[0]);
    // with at least one radix pass, the first pass takes the positions (the identity) and the
    // weights from their sources, so they are not copied here; with none, they are written where
    // the sorted ones belong
    ea.pos = sorted_pos_out && ps.passes == 0 ? reinterpret_cast<uint32_t *>(sorted_pos_out) : nullptr;
    ea.grow = u32(L.grow[0]);
    ea.wgt = weighted && ps.passes == 0 ? u32(L.wgt[0]) : nullptr;
    ea.B = static_cast<uint32_t>(B);
    ea.T = static_cast<uint32_t>(T);
    ea.nbags = static_cast<uint32_t>(T * B);
    if (index_type == DLRM_INDEX_I32)
        DLRM_LAUNCH("expand", k_expand<int32_t>, dim3((ea.nbags + 255) / 256), dim3(256), 0, stream, ea);
    else
        DLRM_LAUNCH("expand", k_expand<int64_t>, dim3((ea.nbags + 255) / 256), dim3(256), 0, stream, ea);

    // K5
    int cur = 0, shift = 0;
    uint32_t *counts = u32(L.counts), *totals = u32(L.totals);
    for (int p = 0; p < ps.passes; ++p) {
        const bool last = p + 1 == ps.passes;
        SortIO io{};
        io.kin = u32(L.keys[cur]);
        io.kout = u32(L.keys[cur ^ 1]);
        // payloads: the grad row, the weight (weighted), the position (only when the sorted
        // positions are an output: the update does not need them)
        int q = 0;
        io.pin[q] = u32(L.grow[cur]);
        io.pout[q++] = u32(L.grow[cur ^ 1]);
        if (weighted) {
            io.pin[q] = p == 0 ? reinterpret_cast<const uint32_t *>(per_sample_weights) : u32(L.wgt[cur]);
            io.pout[q++] = u32(L.wgt[cur ^ 1]);
        }
        if (sorted_pos_out) {
            io.pin[q] = p == 0 ? nullptr : u32(L.pos[cur]);
            io.pout[q++] = last ? reinterpret_cast<uint32_t *>(sorted_pos_out) : u32(L.pos[cur ^ 1]);
        }
        const int NP = q;
        if (ps.rb[p] == 8) launch_radix_pass<8>(io, NP, n, shift, counts, L.nblk, totals, stream);
        else if (ps.rb[p] == 9) launch_radix_pass<9>(io, NP, n, shift, counts, L.nblk, totals, stream);
        else launch_radix_pass<10>(io, NP, n, shift, counts, L.nblk, totals, stream);
        shift += ps.rb[p];
        cur ^= 1;
    }
    const uint32_t *skeys = u32(L.keys[cur]);

    // K6 (always: the update's finisher reads the segment offsets)
    uint32_t *seg_count = u32(L.seg_count);
    int64_t *seg_offsets = segment_offsets_out ? segment_offsets_out : reinterpret_cast<int64_t *>(ws + L.seg_offsets);
    DLRM_LAUNCH("seg_count", k_seg_count, dim3(L.nblk), dim3(256), 0, stream, skeys, n, seg_count);
    DLRM_LAUNCH("seg_write", k_seg_write, dim3(L.nblk), dim3(256), 0, stream, skeys, n, seg_count, L.nblk,
                unique_keys_out, seg_offsets, u32(L.chunk_seg), static_cast<uint32_t>(L.CS), num_unique_out,
                u32(L.fin_count));
    return launch_status();
}

// The update from a planned workspace.  `clear_worklist`: empty the finisher's worklist first
// (not needed right after a plan on the same stream, which leaves it empty).
static int apply_impl(void *const *tables, float *const *state, const int64_t *rows, int32_t T, int32_t D,
                      int32_t dtype, int64_t B, int64_t nnz, int32_t weighted, const float *grad_pooled,
                      int32_t optimizer, float lr, float eps, void *workspace, size_t workspace_bytes,
                      const int64_t *segment_offsets, dlrm_stream_t stream_, bool clear_worklist) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (optimizer != DLRM_OPT_ADAGRAD && optimizer != DLRM_OPT_SGD) return DLRM_ERR_INVALID_ARG;
    int rc = check_rows(rows, T);
    if (rc != DLRM_OK) return rc;
    if (!tables || D < 1 || B < 0 || nnz < 0) return DLRM_ERR_INVALID_ARG;
    if (dtype != DLRM_F32 && dtype != DLRM_BF16) return DLRM_ERR_INVALID_ARG;
    int G, W;
    if (!bwd_geometry(D, &G, &W) || (dtype == DLRM_BF16 && D % 8 != 0)) return DLRM_ERR_UNSUPPORTED;
    if (nnz >= (int64_t(1) << 31) || static_cast<int64_t>(T) * B >= (int64_t(1) << 31)) return DLRM_ERR_UNSUPPORTED;
    const bool adagrad = optimizer == DLRM_OPT_ADAGRAD;
    if (adagrad && !state) return DLRM_ERR_INVALID_ARG;
    for (int t = 0; t < T; ++t) {
        if (!tables[t] || !aligned(tables[t], 16)) return DLRM_ERR_INVALID_ARG;
        if (adagrad && (!state[t] || !aligned(state[t], 4))) return DLRM_ERR_INVALID_ARG;
    }
    if (nnz > 0 && (!grad_pooled || !aligned(grad_pooled, 16))) return DLRM_ERR_INVALID_ARG;
    PlanShape ps;
    rc = plan_shape(rows, T, D, nnz, &ps);
    if (rc != DLRM_OK) return rc;
    const Layout &L = ps.L;
    if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256)) return DLRM_ERR_WORKSPACE;
    if (nnz == 0) return DLRM_OK;
    char *ws = static_cast<char *>(workspace);
    auto u32 = [&](size_t off) { return reinterpret_cast<uint32_t *>(ws + off); };

    // the finisher worklist of this update starts empty (so a plan may be applied more than once)
    if (clear_worklist) DLRM_LAUNCH("zero_u32", k_zero_u32, dim3(1), dim3(1), 0, stream, u32(L.fin_count));
    AdagradArgs a{};
    uint64_t acc_rows = 0;
    for (int t = 0; t < T; ++t) {
        a.tables[t] = static_cast<char *>(tables[t]);
        a.state[t] = adagrad ? state[t] : nullptr;
        a.rowbase[t] = static_cast<uint32_t>(acc_rows);
        acc_rows += static_cast<uint64_t>(rows[t]);
    }
    a.skeys = u32(L.keys[ps.cur]);
    a.sgrow = u32(L.grow[ps.cur]);
    a.swgt = reinterpret_cast<const float *>(u32(L.wgt[ps.cur]));
    a.grad = grad_pooled;
    a.seg_offsets = segment_offsets ? segment_offsets : reinterpret_cast<const int64_t *>(ws + L.seg_offsets);
    a.chunk_seg = u32(L.chunk_seg);
    a.fin_count = u32(L.fin_count);
    a.fin_list = u32(L.fin_list);
    a.part_a = reinterpret_cast<float *>(ws + L.part_a);
    a.part_b = reinterpret_cast<float *>(ws + L.part_b);
    a.n = static_cast<uint32_t>(nnz);
    a.nchunk = L.nchunk;
    a.T = T;
    a.D = D;
    a.divT = make_fastdiv(static_cast<uint32_t>(T));
    a.lr = lr;
    a.eps = eps;
    a.inv_D = 1.0f / static_cast<float>(D);
    const bool w = weighted != 0;
    if (adagrad) {
        if (dtype == DLRM_F32) dispatch_k7<DLRM_F32, DLRM_OPT_ADAGRAD>(a, L.G, L.W, w, L.short_chunks, stream);
        else dispatch_k7<DLRM_BF16, DLRM_OPT_ADAGRAD>(a, L.G, L.W, w, L.short_chunks, stream);
    } else {
        if (dtype == DLRM_F32) dispatch_k7<DLRM_F32, DLRM_OPT_SGD>(a, L.G, L.W, w, L.short_chunks, stream);
        else dispatch_k7<DLRM_BF16, DLRM_OPT_SGD>(a, L.G, L.W, w, L.short_chunks, stream);
    }
    return launch_status();
}

extern "C" int emb_bag_bwd_apply(void *const *tables, float *const *state, const int64_t *rows, int32_t T,
                                 int32_t D, int32_t dtype, int64_t B, int64_t nnz, int32_t weighted,
                                 const float *grad_pooled, int32_t optimizer, float lr, float eps, void *workspace,
                                 size_t workspace_bytes, const int64_t *segment_offsets, dlrm_stream_t stream) {
    return apply_impl(tables, state, rows, T, D, dtype, B, nnz, weighted, grad_pooled, optimizer, lr, eps, workspace,
                      workspace_bytes, segment_offsets, stream, true);
}

extern "C" int emb_bag_bwd_update(void *const *tables, float *const *state, const int64_t *rows,
                                  int32_t T, int32_t D, int32_t dtype, const void *indices,
                                  const void *offsets, int32_t index_type,
                                  const float *per_sample_weights, int64_t B, int64_t nnz,
                                  const float *grad_pooled, int32_t optimizer, float lr, float eps,
                                  void *workspace, size_t workspace_bytes, int64_t *unique_keys_out,
                                  int64_t *segment_offsets_out, int32_t *sorted_pos_out,
                                  int64_t *num_unique_out, uint32_t flags, dlrm_stream_t stream) {
    using namespace dlrm;
    // the update's own checks first, so that an invalid call enqueues nothing
    if (optimizer != DLRM_OPT_ADAGRAD && optimizer != DLRM_OPT_SGD) return DLRM_ERR_INVALID_ARG;
    int rc = check_batch(const_cast<const void *const *>(tables), rows, T, D, dtype, indices, offsets, index_type,
                         per_sample_weights, B, nnz);
    if (rc != DLRM_OK) return rc;
    int G, W;
    if (!bwd_geometry(D, &G, &W) || (dtype == DLRM_BF16 && D % 8 != 0)) return DLRM_ERR_UNSUPPORTED;
    if (optimizer == DLRM_OPT_ADAGRAD) {
        if (!state) return DLRM_ERR_INVALID_ARG;
        for (int t = 0; t < T; ++t)
            if (!state[t] || !aligned(state[t], 4)) return DLRM_ERR_INVALID_ARG;
    }
    if (nnz > 0 && (!grad_pooled || !aligned(grad_pooled, 16))) return DLRM_ERR_INVALID_ARG;
    rc = emb_bag_bwd_plan(rows, T, D, indices, offsets, index_type, per_sample_weights, B, nnz, workspace,
                          workspace_bytes, unique_keys_out, segment_offsets_out, sorted_pos_out, num_unique_out,
                          flags, stream);
    if (rc != DLRM_OK) return rc;
    return apply_impl(tables, state, rows, T, D, dtype, B, nnz, per_sample_weights != nullptr ? 1 : 0, grad_pooled,
                      optimizer, lr, eps, workspace, workspace_bytes, segment_offsets_out, stream, false);
}

extern "C" int emb_bag_bwd_adagrad(void *const *tables, float *const *state, const int64_t *rows,
                                   int32_t T, int32_t D, int32_t dtype, const int64_t *indices,
                                   const int64_t *offsets, const float *per_sample_weights,
                                   int64_t B, int64_t nnz, const float *grad_pooled, float lr,
                                   float eps, void *workspace, size_t workspace_bytes,
                                   int64_t *unique_keys_out, int64_t *segment_offsets_out,
                                   int32_t *sorted_pos_out, int64_t *num_unique_out,
                                   uint32_t flags, dlrm_stream_t stream) {
    return emb_bag_bwd_update(tables, state, rows, T, D, dtype, indices, offsets, DLRM_INDEX_I64,
                              per_sample_weights, B, nnz, grad_pooled, DLRM_OPT_ADAGRAD, lr, eps,
                              workspace, workspace_bytes, unique_keys_out, segment_offsets_out,
                              sorted_pos_out, num_unique_out, flags, stream);
}

// ---------------------------------------------------------------- allocation-free variant
//
// For callers that cannot allocate (code under graph capture, tight serving loops): the same
// plan and update, with the workspace in a fixed array of device memory that the library owns.
// Each GPU the library runs on holds its own copy of the array until the process ends; host code
// reaches it only through the address hipGetSymbolAddress gives on that device (the array's name
// is a host-side stand-in, not a device address).  Calls that overlap on one GPU share the array
// and race.

namespace dlrm {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
}  // namespace dlrm

static __device__ __align__(256) char scratch[dlrm::kScratchBytes];

namespace dlrm {
namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the scratch array, looked up once per device with that device current.
int scratch_on(hipStream_t stream, void **out) {
    hipDevice_t dev = 0;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return DLRM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DLRM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return DLRM_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return DLRM_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return DLRM_ERR_HIP;
        if (e != hipSuccess || !p || !aligned(p, 256)) return DLRM_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DLRM_OK;
}

}  // namespace
}  // namespace dlrm

extern "C" size_t emb_bag_bwd_noalloc_max_bytes(void) { return dlrm::kScratchBytes; }

extern "C" int emb_bag_bwd_update_noalloc(void *const *tables, float *const *state, const int64_t *rows,
                                          int32_t T, int32_t D, int32_t dtype, const void *indices,
                                          const void *offsets, int32_t index_type,
                                          const float *per_sample_weights, int64_t B, int64_t nnz,
                                          const float *grad_pooled, int32_t optimizer, float lr, float eps,
                                          int64_t *unique_keys_out, int64_t *segment_offsets_out,
                                          int32_t *sorted_pos_out, int64_t *num_unique_out, uint32_t flags,
                                          dlrm_stream_t stream_) {
    using namespace dlrm;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    // the batch and size checks first: a batch the scratch cannot hold is refused on the host
    int rc = check_batch(const_cast<const void *const *>(tables), rows, T, D, dtype, indices, offsets, index_type,
                         per_sample_weights, B, nnz);
    if (rc != DLRM_OK) return rc;
    int G, W;
    if (!bwd_geometry(D, &G, &W) || (dtype == DLRM_BF16 && D % 8 != 0)) return DLRM_ERR_UNSUPPORTED;
    PlanShape ps;
    rc = plan_shape(rows, T, D, nnz, &ps);
    if (rc != DLRM_OK) return rc;
    if (ps.L.total > kScratchBytes) return DLRM_ERR_WORKSPACE;
    void *ws = nullptr;
    rc = scratch_on(stream, &ws);
    if (rc != DLRM_OK) return rc;
    return emb_bag_bwd_update(tables, state, rows, T, D, dtype, indices, offsets, index_type, per_sample_weights, B,
                              nnz, grad_pooled, optimizer, lr, eps, ws, kScratchBytes, unique_keys_out,
                              segment_offsets_out, sorted_pos_out, num_unique_out, flags, stream_);
}
