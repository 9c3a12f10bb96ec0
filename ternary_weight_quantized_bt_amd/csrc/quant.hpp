// quant.hpp -- per-token absmax int8 quantization, as device building blocks
// shared by the standalone quantization kernel and the fused prologue of the
// decode kernel, so both produce bit-identical codes.
//
// [PARA] section 5 ("The Mathematics of BitNet b1.58"): activations are
// quantized to 8-bit integers with one AbsMax scale per token (Quant8).  The
// pages print no formula; the one implemented (stated in libternary.h):
//   amax = max|x| (float32; exact in any order), inv = 127 / amax (float32,
//   correctly rounded), xq = clamp(rne(x * inv), -127, 127) with a float32
//   multiply and round-half-to-even, scale = amax, sum = sum of xq.  Where
//   127 / amax overflows, inv = +infinity and the same steps give
//   127 * sign(x) after the clamp, with 0 * infinity taken as 0.
// __fdiv_rn / __fmul_rn / __fadd_rn pin the division, the product and the
// rounding addition whatever the compiler flags (no contraction into fma).
#pragma once

#include "common.hpp"

namespace bt {

// Eight consecutive inputs widened to float32 (bf16 widening is exact).
struct Eight {
    float v[8];
};

__device__ __forceinline__ Eight load8(const float *p) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    return Eight{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}

__device__ __forceinline__ Eight load8(const uint16_t *p) {
    const uint4 a = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    Eight e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e.v[2 * i] = __uint_as_float(w[i] << 16);
        e.v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    return e;
}

// Eight consecutive raw inputs kept in registers between the two halves of a
// one-pass quantization (amax first, codes after the workgroup agrees on it).
template <typename T>
struct Raw8;

// The magnitude of an IEEE value is its bit pattern with the sign cleared,
// and for non-negative values the order of the bit patterns (as unsigned
// integers) is the order of the values.  So max|x| is found exactly with
// integer maxima over the cleared bits (finite inputs only, as the contract
// says); abs_bits() returns that maximum for the eight values of a chunk, in
// float32 bit layout.
template <>
struct Raw8<uint16_t> {
    uint4 a;
    __device__ __forceinline__ void load(const uint16_t *p) {
        const v4u v = *to_global(reinterpret_cast<const v4u *>(p));
        a = make_uint4(v.x, v.y, v.z, v.w);
    }
    __device__ __forceinline__ uint32_t abs_bits() const {
        uint32_t r = 0;
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) r = max(r, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
        return r << 16;
    }
    __device__ __forceinline__ Eight eight() const {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
        Eight e;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e.v[2 * i] = __uint_as_float(w[i] << 16);
            e.v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
        return e;
    }
};

template <>
struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        const gptr<const v4u> q = to_global(reinterpret_cast<const v4u *>(p));
        const v4u u = q[0], v = q[1];
        a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                        __uint_as_float(u.w));
        b = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                        __uint_as_float(v.w));
    }
    __device__ __forceinline__ uint32_t abs_bits() const {
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t r = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) r = max(r, __float_as_uint(v[i]) & 0x7FFFFFFFu);
        return r;
    }
    __device__ __forceinline__ Eight eight() const {
        return Eight{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
    }
};

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
    return v;
}

// 127 / amax, or 0 for an all-zero token (every code is then 0).  amax is
// non-negative; its bits are tested so that a subnormal amax is never taken
// for zero, whatever the denormal mode.
__device__ __forceinline__ float quant_inv(float amax) {
    return __float_as_uint(amax) == 0u ? 0.0f : __fdiv_rn(127.0f, amax);
}

// Round-half-even of x * inv, clamped to [-127, 127], as an int8 code in the
// low byte of the result.  For a finite inv (|x| <= amax, so |x * inv| <=
// 127 * (1 + 2^-24)^2 < 127.5 and the clamp never acts) the product is
// rounded to binary32 first and then 1.5 * 2^23 is added: in that range a
// binary32 addition rounds to an integer, half to even, and leaves it in the
// low mantissa bits, so the low byte of the sum's bits is the code.
__device__ __forceinline__ uint32_t quant1(float x, float inv) {
    return __float_as_uint(__fadd_rn(__fmul_rn(x, inv), 12582912.0f));
}

// The code for an infinite inv (amax below 127 / FLT_MAX): x * inf clamped,
// i.e. 127 * sign(x), and 0 for x == 0 (0 * inf taken as 0).
__device__ __forceinline__ uint32_t quant1_inf(float x) {
    return x > 0.0f ? 127u : (x < 0.0f ? 0xFFFFFF81u : 0u);
}

// Low bytes of four words as one little-endian int8x4 word (v_perm_b32:
// selector bytes 0-3 take bytes of the second operand, 4-7 of the first, 12
// gives zero).
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Pack eight codes (low bytes) into two little-endian int8x4 words; adds
// the codes to `sum` (a signed dot product of each word with ones).
__device__ __forceinline__ uint2 pack8(const uint32_t (&q)[8], int &sum) {
    const uint32_t lo = pack4(q[0], q[1], q[2], q[3]);
    const uint32_t hi = pack4(q[4], q[5], q[6], q[7]);
    sum = __builtin_amdgcn_sdot4((int)lo, 0x01010101, sum, false);
    sum = __builtin_amdgcn_sdot4((int)hi, 0x01010101, sum, false);
    return make_uint2(lo, hi);
}

// Quantize eight values with a finite inv.
__device__ __forceinline__ uint2 quant8_finite(const Eight &e, float inv, int &sum) {
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quant1(e.v[i], inv);
    return pack8(q, sum);
}

// Quantize eight values into two little-endian int8x4 words; adds the codes
// to `sum`.
__device__ __forceinline__ uint2 quant8(const Eight &e, float inv, int &sum) {
    if (__builtin_expect(__builtin_isinf(inv), 0)) {
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = quant1_inf(e.v[i]);
        return pack8(q, sum);
    }
    return quant8_finite(e, inv, sum);
}

// Wave-wide maximum or sum of v, returned to every lane (as a scalar), with
// DPP moves: shifts by 1, 2, 4, 8 lanes within each 16-lane row leave the
// row's result in its lane 15; broadcasts of lane 15 into rows 1 and 3, then
// of lane 31 into rows 2 and 3, leave the wave's result in lane 63.  Lanes a
// move cannot reach contribute the identity (0 for an unsigned max or a sum).
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v) {
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v = MAX ? max(v, t) : v + t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v = MAX ? max(v, t) : v + t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v = MAX ? max(v, t) : v + t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v = MAX ? max(v, t) : v + t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v = MAX ? max(v, t) : v + t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    v = MAX ? max(v, t) : v + t;
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace bt
