// gemv.hip -- decode path for very few tokens: stream the packed weights once
// with 128-bit loads, unpack in registers, int8 dot with v_dot4_i32_i8.
//
// What is computed ([PARA] section 5, figure "BitNet b1.58 Ternary Matrix
// Multiplication": +1 adds the activation, -1 subtracts it, 0 skips it):
//   acc[n,m] = sum_k w[m,k] * xq[n,k] = sum_k code[m,k] * xq[n,k] - xsum[n]
// with code = w + 1 in {0,1,2} ([I2S] "Ternary Representation and
// Packing"), so the codes go straight into the signed dot instruction and
// the per-token code sum is subtracted once at the end.  The pages' CPU
// kernels ([I2S] "How I2_S Kernels Process the Format": weight-parallel and
// activation-parallel SIMD) are prior art; this is a GPU design.
//
// Work split: one workgroup = one 16-row tile of one projection (a grouped
// launch puts q/k/v or gate/up tiles end to end) x NT tokens.  Its waves
// split K into contiguous runs of 256-column blocks; in each block every lane
// loads its 16-byte slot (one 1 KiB tile per wave load, fully coalesced),
// i.e. four words of 16 codes of row r = lane%16 at columns 16*(lane/16) +
// 64*t + 0..15, and dots them with the matching activation words.  Partial
// sums are reduced over the four lanes that share a row (xor-shuffles), then
// over the waves through LDS, and the epilogue dequantizes.

#include "group.hpp"

namespace bt {

namespace {

constexpr int kDot4Waves = 4;
constexpr int kDot4Unroll = 4;

template <int NT>
__device__ __forceinline__ void dot_slot(const uint4 p, const int8_t *x,
                                         int64_t K, int nvalid, int (&acc)[NT]) {
    const uint32_t words[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (j < nvalid) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 xv = *reinterpret_cast<const uint4 *>(x + j * K + 64 * t);
                int s = acc[j];
                s = __builtin_amdgcn_sdot4((int)codes_of_group(words[t], 0), (int)xv.x, s, false);
                s = __builtin_amdgcn_sdot4((int)codes_of_group(words[t], 1), (int)xv.y, s, false);
                s = __builtin_amdgcn_sdot4((int)codes_of_group(words[t], 2), (int)xv.z, s, false);
                s = __builtin_amdgcn_sdot4((int)codes_of_group(words[t], 3), (int)xv.w, s, false);
                acc[j] = s;
            }
        }
    }
}

template <int NT>
__global__ __launch_bounds__(kDot4Waves * kWave)
void gemv_dot4_kernel(GroupArgs a) {
    __shared__ int red[kDot4Waves][NT][16];
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const TileRef tr = resolve_tile(a, blockIdx.x);
    const int64_t n0 = (int64_t)blockIdx.y * NT;
    const int64_t K = a.K;
    const int64_t qb = K / kTileCols;
    const int h = lane / 16;
    const int nvalid = (int)min((int64_t)NT, a.N - n0);

    const uint4 *wp = reinterpret_cast<const uint4 *>(tr.packed + tr.mt * qb * kTileBytes) + lane;
    const int8_t *xb = a.xq + n0 * K + 16 * h;
    const int64_t q0 = qb * wave / kDot4Waves;
    const int64_t q1 = qb * (wave + 1) / kDot4Waves;

    int acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = 0;

    int64_t q = q0;
    for (; q + kDot4Unroll <= q1; q += kDot4Unroll) {
        uint4 p[kDot4Unroll];
#pragma unroll
        for (int u = 0; u < kDot4Unroll; ++u) p[u] = wp[(q + u) * kWave];
#pragma unroll
        for (int u = 0; u < kDot4Unroll; ++u)
            dot_slot<NT>(p[u], xb + (q + u) * kTileCols, K, nvalid, acc);
    }
    for (; q < q1; ++q) dot_slot<NT>(wp[q * kWave], xb + q * kTileCols, K, nvalid, acc);

#pragma unroll
    for (int j = 0; j < NT; ++j) {
        int v = acc[j];
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        if (lane < 16) red[wave][j][lane] = v;
    }
    __syncthreads();
    if (threadIdx.x < 16 * NT) {
        const int j = threadIdx.x / 16, r = threadIdx.x % 16;
        const int64_t n = n0 + j;
        if (n < a.N) {
            int total = 0;
#pragma unroll
            for (int w = 0; w < kDot4Waves; ++w) total += red[w][j][r];
            const float f = token_factor(packed_scale(tr.packed, tr.M, K), a.xs[n]);
            store_out(tr.y, a.ydt, n * tr.M + tr.mt * kTileRows + r, total - a.xsum[n], f);
        }
    }
}

template <int NT>
hipError_t launch_dot4(const GroupArgs &a, hipStream_t s) {
    const dim3 grid((unsigned)group_tiles(a), (unsigned)((a.N + NT - 1) / NT));
    hipLaunchKernelGGL(gemv_dot4_kernel<NT>, grid, dim3(kDot4Waves * kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_decode(const GroupArgs &a, hipStream_t s);

hipError_t launch_decode(const Group &g, hipStream_t s) {
    if (g.N == 0) return hipSuccess;
    const GroupArgs a = make_group_args(g);
    if (g.N == 1) return launch_dot4<1>(a, s);
    if (g.N == 2) return launch_dot4<2>(a, s);
    if (g.N <= kDot4MaxN) return launch_dot4<4>(a, s);
    return launch_mfma_decode(a, s);
}

}  // namespace bt
