// Strict upper triangle of X X^T for a small X (N <= 11 rows) whose columns are split over one
// wavefront: lane l owns columns l*CPL .. l*CPL + CPL - 1 (D = 64 * CPL).  Used by the
// interaction forward and by the fused lookup + interaction, which must agree bit for bit.
//
// Each lane forms its partial dot product of every pair of an 11-row triangle (rows past N are
// zero), then the 64 partials of each pair are summed by recursive halving: at every step a lane
// keeps half of its values, adds its partner's copy of that half, and sends the other half.  The
// two cross-row steps use the gfx950 lane swaps; the four in-row steps use DPP row/half-row
// mirrors and quad permutes (each pairs lanes that differ in the bits not yet decided, so
// partners hold the same pairs).  No step goes through LDS.  Lane p ends with the sum of pair p.
// Every add is of two partial sums in a fixed tree, so the result is deterministic.
#pragma once

#include "common.h"

namespace dlrm {

constexpr int kGramRows = 11;   // N <= 11 (T <= 10 tables)
constexpr int kGramPairs = 55;  // pairs of an 11-row triangle, listed row by row

inline bool gram_ksplit_ok(int N, int D) {
    return N <= kGramRows && (D == 64 || D == 128 || D == 256);
}

template <int CTRL>
__device__ __forceinline__ float gram_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Cross-row halving step on n values with the gfx950 lane swaps: v_permlane32_swap (ROWS = 32)
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes of its second, and
// v_permlane16_swap (ROWS = 16) the odd 16-lane rows of the first with the even rows of the
// second.  Given (lower half, upper half), a lane of the lower group ends with its own lower
// value and its partner's, a lane of the upper group with its partner's upper value and its own,
// so one add finishes the step: lower lanes keep the lower half, upper lanes the upper half.
template <int N_, int ROWS>
__device__ __forceinline__ void gram_halve_swap(float *s) {
    constexpr int H = N_ / 2;
#pragma unroll
    for (int k = 0; k < H; ++k) {
        const uint32_t lo = __float_as_uint(s[k]), hi = __float_as_uint(s[k + H]);
        const auto r = ROWS == 32 ? __builtin_amdgcn_permlane32_swap(lo, hi, false, false)
                                  : __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
        s[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

// In-row halving step on n values through DPP: lanes with `up` set keep the upper half.
template <int N_, int XOR, int DPP_CTRL>
__device__ __forceinline__ void gram_halve(float *s, bool up) {
    constexpr int H = N_ / 2;
#pragma unroll
    for (int k = 0; k < H; ++k) {
        const float send = up ? s[k] : s[k + H];
        const float keep = up ? s[k + H] : s[k];
        float recv;
        if constexpr (DPP_CTRL >= 0) recv = gram_dpp<DPP_CTRL>(send);
        else recv = __shfl_xor(send, XOR);
        s[k] = keep + recv;
    }
}

// x[i][w] = X[i][lane*CPL + w] for i < 11 (zero past N).  Returns the dot product of pair `lane`
// of the 11-row triangle (0 for lanes >= 55).
template <int CPL>
__device__ __forceinline__ float gram_ksplit(const float (&x)[kGramRows][CPL]) {
    float s[64];
    int p = 0;
#pragma unroll
    for (int i = 0; i < kGramRows; ++i)
#pragma unroll
        for (int j = i + 1; j < kGramRows; ++j, ++p) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < CPL; ++w) v = fmaf(x[i][w], x[j][w], v);
            s[p] = v;
        }
#pragma unroll
    for (int k = kGramPairs; k < 64; ++k) s[k] = 0.f;
    const int lane = __lane_id();
    gram_halve_swap<64, 32>(s);  // lanes l, l ^ 32
    gram_halve_swap<32, 16>(s);  // lanes l, l ^ 16
    gram_halve<16, 0, 0x140>(s, lane & 8);  // row_mirror: lane ^ 15 within a row of 16
    gram_halve<8, 0, 0x141>(s, lane & 4);   // row_half_mirror: lane ^ 7 within 8
    gram_halve<4, 0, 0x1B>(s, lane & 2);    // quad_perm [3,2,1,0]: lane ^ 3
    gram_halve<2, 0, 0xB1>(s, lane & 1);    // quad_perm [1,0,3,2]: lane ^ 1
    return s[0];
}

// (i, j) of pair p < 55 of the 11-row triangle; for p >= 55 (lanes holding padding) the loop
// stops at i = 10 and j >= 11, which no caller writes.
__device__ __forceinline__ void gram_pair(int p, int &i, int &j) {
    i = 0;
    while (i < kGramRows - 1 && p >= kGramRows - 1 - i) {
        p -= kGramRows - 1 - i;
        ++i;
    }
    j = i + 1 + p;
}

}  // namespace dlrm
