// quant.hpp -- per-token absmax int8 quantization, as device building blocks
// shared by the standalone quantization kernel and the fused prologue of the
// decode kernel, so both produce bit-identical codes.
//
// [PARA] section 5 ("The Mathematics of BitNet b1.58"): activations are
// quantized to 8-bit integers with one AbsMax scale per token (Quant8).  The
// pages print no formula; the one implemented (stated in libternary.h):
//   amax = max|x| (float32; exact in any order), inv = 127 / amax (float32,
//   correctly rounded), xq = clamp(rne(x * inv), -127, 127) with a float32
//   multiply and round-half-to-even, scale = amax, sum = sum of xq.
// __fdiv_rn / __fmul_rn pin the division and the product whatever the
// compiler flags; rintf is round-half-to-even.
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
        a = *reinterpret_cast<const uint4 *>(p);
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
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
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

// 127 / amax, or 0 for an all-zero token (every code is then 0).
__device__ __forceinline__ float quant_inv(float amax) {
    return amax == 0.0f ? 0.0f : __fdiv_rn(127.0f, amax);
}

__device__ __forceinline__ int quant1(float x, float inv) {
    float r = rintf(__fmul_rn(x, inv));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Quantize eight values into two little-endian int8x4 words; adds the codes
// to `sum`.
__device__ __forceinline__ uint2 quant8(const Eight &e, float inv, int &sum) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int a = quant1(e.v[i], inv);
        const int b = quant1(e.v[4 + i], inv);
        sum += a + b;
        lo |= ((uint32_t)a & 0xFFu) << (8 * i);
        hi |= ((uint32_t)b & 0xFFu) << (8 * i);
    }
    return make_uint2(lo, hi);
}

}  // namespace bt
