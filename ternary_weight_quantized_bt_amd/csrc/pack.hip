// pack.hip -- int8 ternary matrix <-> packed 2-bit "T16Q256" layout.
//
// [I2S] "Ternary Representation and Packing": states -1, 0, +1 are stored as
// the 2-bit integers 0, 1, 2, four to a byte, group g shifted left by 6 - 2g.
// [I2S] "Per-Tensor Scaling Strategy": one float scale after the codes.
// The tile geometry (16 rows x 256 columns per 1 KiB, one 16-byte slot per
// lane of a 64-lane wave) is this library's choice; libternary.h defines it.
//
// One thread builds one 16-byte slot: row m = 16*mt + r, columns
// 256*q + 64*t + 16*h + j for t = 0..3 (one 32-bit word each) and j = 0..15.
// It reads four 16-byte runs of w and writes 16 bytes, so a wave writes one
// whole 1 KiB tile with fully coalesced stores.

#include "common.hpp"
#include "internal.hpp"

namespace bt {

namespace {

constexpr int kPackThreads = 256;

__device__ __forceinline__ uint32_t pack_word(uint4 v, int &bad) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        int val = (int8_t)((in[j >> 2] >> (8 * (j & 3))) & 0xFF);
        if (val < -1) { val = -1; ++bad; }
        if (val > 1) { val = 1; ++bad; }
        const uint32_t code = (uint32_t)(val + 1);
        const int g = j >> 2, i = j & 3;  // column 4g + i of the word
        word |= code << (8 * i + 6 - 2 * g);
    }
    return word;
}

__global__ __launch_bounds__(kPackThreads)
void pack_kernel(const int8_t *__restrict__ w, int64_t M, int64_t K,
                 float scale, uint8_t *__restrict__ packed,
                 int32_t *__restrict__ invalid) {
    const int64_t qb = K / kTileCols;
    const int64_t nslots = (M / kTileRows) * qb * kWave;
    const int64_t slot = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    int bad = 0;
    if (slot < nslots) {
        const int64_t tile = slot / kWave;
        const int lane = (int)(slot % kWave);
        const int64_t mt = tile / qb, q = tile % qb;
        const int r = lane % 16, h = lane / 16;
        const int8_t *src = w + (mt * kTileRows + r) * K + q * kTileCols + 16 * h;
        uint4 out;
        out.x = pack_word(*reinterpret_cast<const uint4 *>(src + 0), bad);
        out.y = pack_word(*reinterpret_cast<const uint4 *>(src + 64), bad);
        out.z = pack_word(*reinterpret_cast<const uint4 *>(src + 128), bad);
        out.w = pack_word(*reinterpret_cast<const uint4 *>(src + 192), bad);
        reinterpret_cast<uint4 *>(packed)[slot] = out;
    }
    if (invalid != nullptr) {
        const int total = wave_sum(bad);
        if ((threadIdx.x % kWave) == 0 && total != 0) atomicAdd(invalid, total);
    }
    // Tail: the scale, then zeros up to 256 bytes.
    if (blockIdx.x == 0 && threadIdx.x < BT_TAIL_BYTES / 4) {
        uint32_t *tail = reinterpret_cast<uint32_t *>(packed + M * K / 4);
        tail[threadIdx.x] = threadIdx.x == 0 ? __float_as_uint(scale) : 0u;
    }
}

__global__ __launch_bounds__(kPackThreads)
void unpack_kernel(const uint8_t *__restrict__ packed, int64_t M, int64_t K,
                   int8_t *__restrict__ w) {
    const int64_t qb = K / kTileCols;
    const int64_t nslots = (M / kTileRows) * qb * kWave;
    const int64_t slot = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
    if (slot >= nslots) return;
    const int64_t tile = slot / kWave;
    const int lane = (int)(slot % kWave);
    const int64_t mt = tile / qb, q = tile % qb;
    const int r = lane % 16, h = lane / 16;
    int8_t *dst = w + (mt * kTileRows + r) * K + q * kTileCols + 16 * h;
    const uint4 p = reinterpret_cast<const uint4 *>(packed)[slot];
    const uint32_t words[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t c = codes_of_group(words[t], g);  // byte i = col 4g+i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t code = (c >> (8 * i)) & 0xFFu;
                const uint32_t val = (uint32_t)(uint8_t)(int8_t)((int)code - 1);
                o[g] |= val << (8 * i);
            }
        }
        *reinterpret_cast<uint4 *>(dst + 64 * t) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

hipError_t launch_pack(const int8_t *w, int64_t M, int64_t K, float scale,
                       uint8_t *packed, int32_t *invalid, hipStream_t s) {
    const int64_t nslots = (M / kTileRows) * (K / kTileCols) * kWave;
    const int64_t blocks = (nslots + kPackThreads - 1) / kPackThreads;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(kPackThreads),
                       0, s, w, M, K, scale, packed, invalid);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int64_t M, int64_t K,
                         int8_t *w, hipStream_t s) {
    const int64_t nslots = (M / kTileRows) * (K / kTileCols) * kWave;
    const int64_t blocks = (nslots + kPackThreads - 1) / kPackThreads;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(kPackThreads),
                       0, s, packed, M, K, w);
    return hipGetLastError();
}

}  // namespace bt
