// dot4.hpp -- the single-token inner step: one 16-byte packed slot (64 codes
// of one row) dotted with the matching int8 activations of up to NT tokens
// with v_dot4_i32_i8, shared by the per-group and the per-layer kernels.
//
// What is computed ([PARA] section 5, figure "BitNet b1.58 Ternary Matrix
// Multiplication"): sum_k code[m,k] * xq[n,k], code = w + 1 in {0,1,2}
// ([I2S] "Ternary Representation and Packing"); the token's code sum is
// subtracted once at the end.
//
// Unpacking: a word's group g holds its codes at bits 8i + 6 - 2g.  Groups
// 1..3 are used in place, masked but not shifted, so their bytes are
// code << 4, code << 2 and code (all <= 32: valid signed int8 operands) and
// are summed into accumulators of weight 16, 4 and 1; group 0 is shifted
// down.  The weighted sums are exact multiples of 16 and 4 and are shifted
// back before the reduction (acc_total).
#pragma once

#include "common.hpp"

namespace bt {

// Per-token accumulators of the three code weights.
template <int NT>
struct Acc {
    int a1[NT];   // weight 1: groups 0 and 3
    int a4[NT];   // weight 4: group 2
    int a16[NT];  // weight 16: group 1
};

template <int NT>
__device__ __forceinline__ void acc_zero(Acc<NT> &c) {
#pragma unroll
    for (int j = 0; j < NT; ++j) c.a1[j] = c.a4[j] = c.a16[j] = 0;
}

// Adds the dot products of one 16-byte slot (64 codes of one row) with the
// matching activations of tokens j < nvalid (rows of x are K bytes apart).
template <int NT>
__device__ __forceinline__ void dot_slot(const v4u p, const int8_t *x, int64_t K,
                                         int nvalid, Acc<NT> &c) {
    const uint32_t words[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t w = words[t];
        const int g0 = (int)((w >> 6) & kCodeMask);  // code
        const int g1 = (int)(w & (kCodeMask << 4));  // code << 4
        const int g2 = (int)(w & (kCodeMask << 2));  // code << 2
        const int g3 = (int)(w & kCodeMask);         // code
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j >= nvalid) break;
            const uint4 xv = *reinterpret_cast<const uint4 *>(x + j * K + 64 * t);
            int s1 = c.a1[j];
            s1 = __builtin_amdgcn_sdot4(g0, (int)xv.x, s1, false);
            s1 = __builtin_amdgcn_sdot4(g3, (int)xv.w, s1, false);
            c.a1[j] = s1;
            c.a16[j] = __builtin_amdgcn_sdot4(g1, (int)xv.y, c.a16[j], false);
            c.a4[j] = __builtin_amdgcn_sdot4(g2, (int)xv.z, c.a4[j], false);
        }
    }
}

// a1 + a4/4 + a16/16 for token j: this lane's share of the row's sum.
template <int NT>
__device__ __forceinline__ int acc_total(const Acc<NT> &c, int j) {
    return c.a1[j] + (c.a4[j] >> 2) + (c.a16[j] >> 4);
}

}  // namespace bt
