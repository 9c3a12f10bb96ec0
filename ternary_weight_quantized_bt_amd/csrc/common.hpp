// common.hpp -- device helpers shared by the libternary kernels (gfx950).
//
// Pages cited:
//   [I2S]  "How BitNet's 1-Bit (I2_S) Quantization Works Compared to Standard
//          LLM Quantization"
//   [PARA] "LLM Quantization Paradigms: FP8, AWQ, EXL2 & BitNet b1.58 in 2026"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libternary.h"

namespace bt {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Pointers into global memory.  Loads through them compile to global_load
// (counted by vmcnt only) rather than flat_load, whose lgkmcnt side would make
// every LDS wait also drain the in-flight HBM loads.
template <typename T>
using gptr = __attribute__((address_space(1))) T *;

template <typename T>
__device__ __forceinline__ gptr<T> to_global(T *p) {
    return (gptr<T>)p;
}

constexpr int kWave = 64;
constexpr int kTileRows = 16;     // rows of one packed tile
constexpr int kTileCols = 256;    // columns of one packed tile
constexpr int kTileBytes = 1024;  // 16 x 256 codes at 2 bits
constexpr uint32_t kCodeMask = 0x03030303u;

// Codes of the four 4-column groups of one packed 32-bit word.  Word bit
// 8*i + 6 - 2*g holds the code of column 4*g + i ([I2S] "Ternary
// Representation and Packing": group g is shifted left by 6 - 2g inside its
// byte), so shifting right by 6 - 2g and masking two bits per byte yields a
// word whose byte i is the code (0, 1, 2) of column 4*g + i -- directly an
// int8x4 operand for the dot and matrix-core instructions.
__device__ __forceinline__ uint32_t codes_of_group(uint32_t word, int g) {
    return (word >> (6 - 2 * g)) & kCodeMask;
}

// Round-to-nearest-even float32 -> bfloat16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two float32 -> two bfloat16 (round to nearest even) in one word, low half
// first: gfx950's packed conversion (v_cvt_pk_bf16_f32), the same bits as
// f32_to_bf16 for finite inputs.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    const bf16x2 b = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    uint32_t u;
    __builtin_memcpy(&u, &b, 4);
    return u;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Per-token dequantization factor s_w * s_a / 127 in float32 ([I2S] "How
// I2_S Kernels Process the Format": one per-tensor scale; [PARA] section 5:
// the per-token absmax scale maps 127 to amax).
__device__ __forceinline__ float token_factor(float s_w, float s_a) {
    return __fdiv_rn(__fmul_rn(s_w, s_a), 127.0f);
}

// Store one output: the exact integer sum, or its dequantized value.
__device__ __forceinline__ void store_out(void *y, int ydt, int64_t idx,
                                          int32_t acc, float factor) {
    if (ydt == BT_I32) {
        to_global(reinterpret_cast<int32_t *>(y))[idx] = acc;
    } else {
        float v = __fmul_rn((float)acc, factor);
        if (ydt == BT_F32)
            to_global(reinterpret_cast<float *>(y))[idx] = v;
        else
            to_global(reinterpret_cast<uint16_t *>(y))[idx] = f32_to_bf16(v);
    }
}

// Store four consecutive outputs y[idx .. idx+3] (idx a multiple of 4) with
// one vector store: acc[v] - sub, dequantized by `factor` unless BT_I32.
__device__ __forceinline__ void store_out4(void *y, int ydt, int64_t idx, const v4i acc,
                                           int32_t sub, float factor) {
    if (ydt == BT_I32) {
        *to_global(reinterpret_cast<v4i *>(reinterpret_cast<int32_t *>(y) + idx)) =
            v4i{acc.x - sub, acc.y - sub, acc.z - sub, acc.w - sub};
        return;
    }
    const float v0 = __fmul_rn((float)(acc.x - sub), factor);
    const float v1 = __fmul_rn((float)(acc.y - sub), factor);
    const float v2 = __fmul_rn((float)(acc.z - sub), factor);
    const float v3 = __fmul_rn((float)(acc.w - sub), factor);
    if (ydt == BT_F32) {
        *to_global(reinterpret_cast<v4u *>(reinterpret_cast<float *>(y) + idx)) =
            v4u{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)};
    } else {
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        *to_global(reinterpret_cast<v2u *>(reinterpret_cast<uint16_t *>(y) + idx)) =
            v2u{f32x2_to_bf16x2(v0, v1), f32x2_to_bf16x2(v2, v3)};
    }
}

__device__ __forceinline__ float packed_scale(const uint8_t *packed,
                                              int64_t M, int64_t K) {
    return *to_global(reinterpret_cast<const float *>(packed + M * K / 4));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

}  // namespace bt
