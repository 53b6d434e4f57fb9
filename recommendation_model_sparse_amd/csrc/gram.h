// Strict upper triangle of X X^T for a small X (N <= 11 rows) whose columns are split over one
// wavefront: lane l owns columns l*CPL .. l*CPL + CPL - 1 (D = 64 * CPL).  Used by the
// interaction forward and by the fused lookup + interaction, which must agree bit for bit.
//
// The triangle is that of NR rows (9 for N <= 9, else 11; rows past N are zero).  Each lane forms
// its partial dot product of every pair, then the 64 partials of each pair are summed by
// recursive halving: at every step a lane keeps half of its values (the upper half if its bit of
// the step is set, the half rounded up, padded with zeros), adds its partner's copy of that half,
// and sends the other half.  The two cross-row steps use the gfx950 lane swaps; the four in-row
// steps use DPP row/half-row mirrors and quad permutes (each pairs lanes that differ in the bits
// not yet decided, so partners hold the same pairs).  No step goes through LDS.  After the six
// steps a lane holds the sum of one pair, or only padding (gram_lane_pair says which).  Every add
// is of two partial sums in a fixed tree, so the result is deterministic.
#pragma once

#include "common.h"

namespace dlrm {

constexpr int kGramMaxRows = 11;  // N <= 11 (T <= 10 tables)

inline bool gram_ksplit_ok(int N, int D) {
    return N <= kGramMaxRows && (D == 64 || D == 128 || D == 256);
}

// Rows of the triangle the k-split Gram forms for N vectors.
__host__ __device__ constexpr int gram_rows(int N) { return N <= 9 ? 9 : 11; }

// Values per lane after each of the six halving steps, for P pairs.
__host__ __device__ constexpr int gram_half(int c) { return (c + 1) / 2; }
template <int NR>
struct GramSteps {
    static constexpr int P = NR * (NR - 1) / 2;
    static constexpr int C1 = gram_half(P), C2 = gram_half(C1), C3 = gram_half(C2), C4 = gram_half(C3),
                         C5 = gram_half(C4), C6 = gram_half(C5);
    static_assert(P <= 64 && C6 == 1, "six halvings leave one value per lane");
};

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

// s[from .. to) = 0: the padding of a half that was rounded up.
template <int FROM, int TO>
__device__ __forceinline__ void gram_pad(float *s) {
#pragma unroll
    for (int k = FROM; k < TO; ++k) s[k] = 0.f;
}

// x[i][w] = X[i][lane*CPL + w] for i < NR (zero past N).  Returns this lane's pair sum (see
// gram_lane_pair), or 0 for a lane holding only padding.
template <int NR, int CPL>
__device__ __forceinline__ float gram_ksplit(const float (&x)[NR][CPL]) {
    using G = GramSteps<NR>;
    float s[2 * G::C1];
    int p = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
        for (int j = i + 1; j < NR; ++j, ++p) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < CPL; ++w) v = fmaf(x[i][w], x[j][w], v);
            s[p] = v;
        }
    gram_pad<G::P, 2 * G::C1>(s);
    const int lane = __lane_id();
    gram_halve_swap<2 * G::C1, 32>(s);  // lanes l, l ^ 32
    gram_pad<G::C1, 2 * G::C2>(s);
    gram_halve_swap<2 * G::C2, 16>(s);  // lanes l, l ^ 16
    gram_pad<G::C2, 2 * G::C3>(s);
    gram_halve<2 * G::C3, 0, 0x140>(s, lane & 8);  // row_mirror: lane ^ 15 within a row of 16
    gram_pad<G::C3, 2 * G::C4>(s);
    gram_halve<2 * G::C4, 0, 0x141>(s, lane & 4);  // row_half_mirror: lane ^ 7 within 8
    gram_pad<G::C4, 2 * G::C5>(s);
    gram_halve<2 * G::C5, 0, 0x1B>(s, lane & 2);   // quad_perm [3,2,1,0]: lane ^ 3
    gram_pad<G::C5, 2 * G::C6>(s);
    gram_halve<2 * G::C6, 0, 0xB1>(s, lane & 1);   // quad_perm [1,0,3,2]: lane ^ 1
    return s[0];
}

// The pair (i, j) whose sum gram_ksplit<NR> leaves in this lane, following the halves the lane
// kept (bit 5 of the lane at the first step .. bit 0 at the last); false for a lane that kept
// only padding.  Pairs are numbered row by row over the NR-row triangle.
template <int NR>
__device__ __forceinline__ bool gram_lane_pair(int lane, int &i, int &j) {
    using G = GramSteps<NR>;
    const int C[6] = {G::C1, G::C2, G::C3, G::C4, G::C5, G::C6};
    int p = 0, real = G::P;  // index of the lane's first value; real values among its half
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        if ((lane >> (5 - k)) & 1) {
            p += C[k];
            real = real > C[k] ? real - C[k] : 0;
        } else {
            real = real < C[k] ? real : C[k];
        }
    }
    i = 0;
    while (i < NR - 1 && p >= NR - 1 - i) {
        p -= NR - 1 - i;
        ++i;
    }
    j = i + 1 + p;
    return real >= 1;
}

}  // namespace dlrm
