// mfma.hip -- int8 matrix-core product for more than a handful of tokens.
//
// The ternary contraction ([PARA] section 5, figure "BitNet b1.58 Ternary
// Matrix Multiplication") is a dense int8 contraction once the codes
// 0/1/2 ([I2S] "Ternary Representation and Packing") are unpacked, so it runs
// on v_mfma_i32_16x16x64_i8: acc = sum code*xq over 64 columns per
// instruction, minus the token's code sum at the end.
//
// Operand mapping.  A 16-byte packed slot of lane l holds, in word t, the
// codes of row l%16 at columns 64*t + 16*(l/16) + 0..15; unpacking one word
// gives exactly the 16 int8 A-operand bytes that lane contributes to a
// 16x16x64 instruction over the 64 columns 64*t..64*t+63.  The B operand of
// lane l is the 16 int8 activations of token l%16 at the same 16 columns.
// Because A and B of a lane then cover the same columns in the same byte
// order, the instruction sums over exactly those 64 columns whatever order
// the hardware gives the lane groups.  The 16x16 result lands as: lane l,
// register v = row 4*(l/16) + v, token l%16.

#include "group.hpp"

namespace bt {

namespace {

__device__ __forceinline__ v4i unpack_a(uint32_t word) {
    v4i a;
    a.x = (int)codes_of_group(word, 0);
    a.y = (int)codes_of_group(word, 1);
    a.z = (int)codes_of_group(word, 2);
    a.w = (int)codes_of_group(word, 3);
    return a;
}

// Each wave owns one 16-row tile and 16*TG tokens; the K loop streams the
// tile's packed row once and reads activations straight from global memory.
template <int WAVES, int TG>
__global__ __launch_bounds__(WAVES * kWave)
void mfma_simple_kernel(GroupArgs a) {
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t tile = (int64_t)blockIdx.x * WAVES + wave;
    if (tile >= group_tiles(a)) return;  // whole wave
    const TileRef tr = resolve_tile(a, tile);
    const int64_t K = a.K, qb = K / kTileCols;
    const int r = lane % 16, h = lane / 16;
    const int64_t nb = (int64_t)blockIdx.y * 16 * TG;
    gptr<const v4u> wp = to_global(reinterpret_cast<const v4u *>(tr.packed + tr.mt * qb * kTileBytes)) + lane;

    v4i acc[TG];
#pragma unroll
    for (int g = 0; g < TG; ++g) acc[g] = v4i{0, 0, 0, 0};

    for (int64_t q = 0; q < qb; ++q) {
        const v4u p = wp[q * kWave];
        const uint32_t words[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v4i A = unpack_a(words[t]);
#pragma unroll
            for (int g = 0; g < TG; ++g) {
                const int64_t n = nb + 16 * g + r;
                v4i B = v4i{0, 0, 0, 0};
                if (n < a.N)
                    B = *reinterpret_cast<const v4i *>(a.xq + n * K + q * kTileCols + 64 * t + 16 * h);
                acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, acc[g], 0, 0, 0);
            }
        }
    }

    const float s_w = packed_scale(tr.packed, tr.M, K);
#pragma unroll
    for (int g = 0; g < TG; ++g) {
        const int64_t n = nb + 16 * g + r;
        if (n < a.N) {
            const float f = token_factor(s_w, a.xs[n]);
            const int32_t sub = a.xsum[n];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = tr.mt * kTileRows + 4 * h + v;
                store_out(tr.y, a.ydt, n * tr.M + m, acc[g][v] - sub, f);
            }
        }
    }
}

template <int WAVES, int TG>
hipError_t launch_simple(const GroupArgs &a, hipStream_t s) {
    const int64_t tiles = group_tiles(a);
    const dim3 grid((unsigned)((tiles + WAVES - 1) / WAVES),
                    (unsigned)((a.N + 16 * TG - 1) / (16 * TG)));
    hipLaunchKernelGGL((mfma_simple_kernel<WAVES, TG>), grid, dim3(WAVES * kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_decode(const GroupArgs &a, hipStream_t s) {
    return launch_simple<4, 4>(a, s);
}


}  // namespace bt
