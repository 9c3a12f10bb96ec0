// interop.hip -- dequantization of packed weights (to_float) and conversion
// between the T16Q256 layout and the I2_S byte layout.
//
// "ik_llama.cpp 运行 BitNet b1.58 2B 模型实战…", section 5.1: an I2_S tensor
// is turned back into float32 as a whole (to_float) before requantization.
// "How BitNet's 1-Bit (I2_S) Quantization Works Compared to Standard LLM
// Quantization", "Ternary Representation and Packing": codes 0, 1, 2 for
// -1, 0, +1, shifted left by 6 - 2 * group inside a byte, in blocks of
// QK_I2_S weights (a size the page does not give, so it is the caller's
// `block`); "Per-Tensor Scaling Strategy": one float after the codes.
//
// I2_S reading (libternary.h states it for callers): the M*K weights in
// row-major order are cut into blocks of `block`; weight j of a block has
// group g = j / (block/4) and byte j % (block/4) of the block's block/4
// bytes; the float32 scale follows the M*K/4 code bytes.
//
// These are offline conversions: simple one-thread-per-output kernels, the
// I2_S side addressed element by element with incremental block arithmetic.

#include "common.hpp"
#include "internal.hpp"

namespace bt {

namespace {

constexpr int kIoThreads = 256;

// Slot geometry shared by the T16Q256 kernels: thread -> (row, first column
// of its four 16-column runs).
struct SlotPos {
    int64_t row, col0;  // run t covers columns col0 + 64 t .. + 15
};
__device__ __forceinline__ SlotPos slot_pos(int64_t slot, int64_t K) {
    const int64_t qb = K / kTileCols;
    const int64_t tile = slot / kWave;
    const int lane = (int)(slot % kWave);
    const int64_t mt = tile / qb, q = tile % qb;
    return {mt * kTileRows + lane % 16, q * kTileCols + 16 * (lane / 16)};
}

// ---------------------------------------------------------------- to_float

template <typename T>
__global__ __launch_bounds__(kIoThreads)
void dequant_kernel(const uint8_t *__restrict__ packed, int64_t M, int64_t K,
                    T *__restrict__ w) {
    const int64_t nslots = (M / kTileRows) * (K / kTileCols) * kWave;
    const int64_t slot = (int64_t)blockIdx.x * kIoThreads + threadIdx.x;
    if (slot >= nslots) return;
    const float s = packed_scale(packed, M, K);
    const SlotPos sp = slot_pos(slot, K);
    const v4u p = *to_global(reinterpret_cast<const v4u *>(packed) + slot);
    const uint32_t words[4] = {p.x, p.y, p.z, p.w};
    // (code - 1) * s for the three codes: float32 products (exact: -s, a
    // signed zero, s), then rounded to bfloat16 for a bf16 output
    const float f[3] = {__fmul_rn(-1.0f, s), __fmul_rn(0.0f, s), s};
    T vals[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        if constexpr (sizeof(T) == 4) vals[i] = __float_as_uint(f[i]);
        else vals[i] = f32_to_bf16(f[i]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        T out[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const uint32_t code = (words[t] >> (8 * (c & 3) + 6 - 2 * (c >> 2))) & 3u;
            out[c] = code == 0u ? vals[0] : (code == 1u ? vals[1] : vals[2]);
        }
        T *dst = w + sp.row * K + sp.col0 + 64 * t;
        constexpr int kVec = 16 / sizeof(T);  // elements per 16-byte store
#pragma unroll
        for (int v = 0; v < 16 / kVec; ++v) {
            v4u chunk;
            __builtin_memcpy(&chunk, out + v * kVec, 16);
            *to_global(reinterpret_cast<v4u *>(dst + v * kVec)) = chunk;
        }
    }
}

// ------------------------------------------------------------- I2_S import

// Position of element e in the I2_S code bytes, advanced one element at a
// time: block b, group g, byte p within the block's q = block/4 bytes.
struct I2sCursor {
    int64_t b;
    uint32_t g, p, q;
    __device__ void start(int64_t e, int64_t block) {
        q = (uint32_t)(block / 4);
        b = e / block;
        const uint32_t j = (uint32_t)(e - b * block);
        g = j / q;
        p = j - g * q;
    }
    __device__ int64_t byte() const { return b * q + p; }
    __device__ uint32_t shift() const { return 6u - 2u * g; }
    __device__ void next() {
        if (++p == q) {
            p = 0;
            if (++g == 4u) {
                g = 0;
                ++b;
            }
        }
    }
};

__global__ __launch_bounds__(kIoThreads)
void i2s_import_kernel(const uint8_t *__restrict__ src, int64_t M, int64_t K, int64_t block,
                       uint8_t *__restrict__ packed, int32_t *__restrict__ invalid) {
    const int64_t nslots = (M / kTileRows) * (K / kTileCols) * kWave;
    const int64_t slot = (int64_t)blockIdx.x * kIoThreads + threadIdx.x;
    int bad = 0;
    if (slot < nslots) {
        const SlotPos sp = slot_pos(slot, K);
        uint32_t words[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            I2sCursor cur;
            cur.start(sp.row * K + sp.col0 + 64 * t, block);
            uint32_t word = 0;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                uint32_t code = ((uint32_t)src[cur.byte()] >> cur.shift()) & 3u;
                if (code == 3u) {
                    code = 2u;
                    ++bad;
                }
                word |= code << (8 * (c & 3) + 6 - 2 * (c >> 2));
                cur.next();
            }
            words[t] = word;
        }
        *to_global(reinterpret_cast<v4u *>(packed) + slot) = v4u{words[0], words[1], words[2], words[3]};
    }
    if (invalid != nullptr) {
        const int total = wave_sum(bad);
        if ((threadIdx.x % kWave) == 0 && total != 0) atomicAdd(invalid, total);
    }
    if (blockIdx.x == 0 && threadIdx.x < BT_TAIL_BYTES / 4) {
        const uint32_t s = *reinterpret_cast<const uint32_t *>(src + M * K / 4);
        reinterpret_cast<uint32_t *>(packed + M * K / 4)[threadIdx.x] = threadIdx.x == 0 ? s : 0u;
    }
}

// ------------------------------------------------------------- I2_S export

// Code of W[m, k] in the T16Q256 layout.
__device__ __forceinline__ uint32_t t16q256_code(const uint8_t *packed, int64_t K, int64_t m,
                                                 int64_t k) {
    const int64_t tile = (m / kTileRows) * (K / kTileCols) + k / kTileCols;
    const int kk = (int)(k % kTileCols);
    const int slot = (int)(m % kTileRows) + 16 * ((kk % 64) / 16);
    const int64_t off = tile * kTileBytes + slot * 16 + 4 * (kk / 64) + (kk % 4);
    return ((uint32_t)packed[off] >> (6 - 2 * ((kk % 16) / 4))) & 3u;
}

// One thread per 4 consecutive I2_S code bytes.
__global__ __launch_bounds__(kIoThreads)
void i2s_export_kernel(const uint8_t *__restrict__ packed, int64_t M, int64_t K, int64_t block,
                       uint8_t *__restrict__ dst) {
    const int64_t nbytes = M * K / 4;
    const int64_t B0 = 4 * ((int64_t)blockIdx.x * kIoThreads + threadIdx.x);
    if (B0 < nbytes) {
        const int64_t q = block / 4;
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t B = B0 + i;
            const int64_t b = B / q, p = B - (B / q) * q;
            uint32_t byte = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t e = b * block + g * q + p;
                const int64_t m = e / K;
                byte |= t16q256_code(packed, K, m, e - m * K) << (6 - 2 * g);
            }
            out |= byte << (8 * i);
        }
        *to_global(reinterpret_cast<uint32_t *>(dst + B0)) = out;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *reinterpret_cast<uint32_t *>(dst + nbytes) =
            *reinterpret_cast<const uint32_t *>(packed + nbytes);
}

unsigned blocks_for(int64_t threads) {
    return (unsigned)((threads + kIoThreads - 1) / kIoThreads);
}

}  // namespace

hipError_t launch_dequant(const uint8_t *packed, int64_t M, int64_t K, void *w, bt_dtype wdt,
                          hipStream_t s) {
    const int64_t nslots = (M / kTileRows) * (K / kTileCols) * kWave;
    if (wdt == BT_F32)
        hipLaunchKernelGGL(dequant_kernel<uint32_t>, dim3(blocks_for(nslots)), dim3(kIoThreads),
                           0, s, packed, M, K, static_cast<uint32_t *>(w));
    else
        hipLaunchKernelGGL(dequant_kernel<uint16_t>, dim3(blocks_for(nslots)), dim3(kIoThreads),
                           0, s, packed, M, K, static_cast<uint16_t *>(w));
    return hipGetLastError();
}

hipError_t launch_i2s_import(const uint8_t *src, int64_t M, int64_t K, int64_t block,
                             uint8_t *packed, int32_t *invalid, hipStream_t s) {
    const int64_t nslots = (M / kTileRows) * (K / kTileCols) * kWave;
    hipLaunchKernelGGL(i2s_import_kernel, dim3(blocks_for(nslots)), dim3(kIoThreads), 0, s,
                       src, M, K, block, packed, invalid);
    return hipGetLastError();
}

hipError_t launch_i2s_export(const uint8_t *packed, int64_t M, int64_t K, int64_t block,
                             uint8_t *dst, hipStream_t s) {
    hipLaunchKernelGGL(i2s_export_kernel, dim3(blocks_for(M * K / 16)), dim3(kIoThreads), 0, s,
                       packed, M, K, block, dst);
    return hipGetLastError();
}

}  // namespace bt
