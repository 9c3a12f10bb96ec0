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
// Persistent grid.  Each workgroup first stages the int8 activations of all
// tokens in LDS -- either by quantizing the float input itself (fused
// prologue, used by the layer driver: no separate quantization launch; one
// pass over the input, kept in registers between the amax reduction and the
// rounding) or by copying already quantized codes -- and then walks the
// 16-row tiles of the group (q/k/v or gate/up tiles laid end to end) with a
// stride of the grid size.  Within a tile its waves split K into contiguous
// runs of 256-column blocks.  In each block a lane loads its 16-byte slot (a
// wave load covers one 1 KiB tile, fully coalesced): four words of 16 codes of
// row lane%16 at columns 16*(lane/16) + 64*t + 0..15, dotted with activation
// words read from LDS (16 lanes read the same address: a broadcast).
//
// Each wave keeps kRing slot loads in flight at all times: a ring of
// registers refilled as it is consumed, running straight across tile
// boundaries, so HBM keeps streaming while a tile is reduced.  The loads are
// non-temporal (every weight byte is read once; 14 % more bandwidth on a
// long stream than ordinary loads).  Sums are
// reduced over the four lanes that share a row (xor-shuffles), then over the
// waves through LDS (double-buffered: one barrier per tile), and the epilogue
// dequantizes.  The first ring fill is issued before the prologue so its HBM
// latency overlaps the activation staging.
//
// Unpacking: a word's group g holds its codes at bits 8i + 6 - 2g.  Groups
// 1..3 are used in place, masked but not shifted, so their bytes are
// code << 4, code << 2 and code (all <= 32: valid signed int8 operands) and
// are summed into accumulators of weight 16, 4 and 1; group 0 is shifted
// down.  The weighted sums are exact multiples of 16 and 4 and are shifted
// back before the reduction.

#include "dot4.hpp"
#include "group.hpp"
#include "quant.hpp"

namespace bt {

namespace {

// Default launch shape: 8 waves per workgroup, each tile split along K over
// kDecSplit waves, kRing slot loads in flight per wave, kDecPerCu
// workgroups per compute unit.
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kDecSplit = 8;
constexpr int kRing = 4;
constexpr int kDecPerCu = 2;
// Activations are staged in LDS when NT*K fits in this many bytes; longer
// rows are read from global memory (already quantized).
constexpr int64_t kDecLdsMax = 64 * 1024;
// Registers (16-byte units per thread) that hold the raw input of a fused
// prologue between its two halves.
constexpr int kRawUnits = 8;

// This lane's 16 bytes of block q of the row tile tr.
__device__ __forceinline__ gptr<const v4u> slot_ptr(const TileRef &tr, int64_t qb, int64_t q,
                                                     int lane) {
    return to_global(reinterpret_cast<const v4u *>(tr.packed + (tr.mt * qb + q) * kTileBytes)) +
           lane;
}

// Activation source of the decode kernel.
struct DecodeX {
    const void *x;        // fused: float / bf16 input [N, K]
    const int8_t *xq;     // not fused: codes [N, K]
    const float *xs;      // not fused: scales [N]
    const int32_t *xsum;  // not fused: code sums [N]
};

// MODE 0: quantize x (element type T) in the prologue, codes into LDS.
// MODE 1: copy pre-quantized codes into LDS.
// MODE 2: read pre-quantized codes from global memory (rows too long for LDS).
//
// WAVES waves per workgroup; each 16-row tile is split along K over P waves
// (P divides WAVES), so a workgroup works on WAVES/P tiles at a time.  With
// P == 1 a wave owns whole tiles and reduces them without any barrier.
template <typename T, int NT, int MODE, int WAVES, int P, int RING>
__global__ __launch_bounds__(WAVES * kWave)
void decode_dot4_kernel(GroupArgs a, DecodeX dx) {
    static_assert(WAVES % P == 0, "K split must divide the waves");
    constexpr int kThreads = WAVES * kWave;
    constexpr int TPW = WAVES / P;  // tiles per workgroup iteration
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    __shared__ int red[P > 1 ? 2 : 1][P > 1 ? WAVES : 1][NT][16];
    __shared__ uint32_t s_amax[WAVES][NT];  // max |x| bits
    __shared__ int s_sum[WAVES][NT];
    __shared__ float s_scale[NT];          // per-token activation scale
    __shared__ int s_xsum[NT];             // per-token code sum
    __shared__ float s_wscale[kMaxGroup];  // per-projection weight scale
    __shared__ float s_factor[kMaxGroup][NT];  // s_w * s_a / 127

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t K = a.K, qb = K / kTileCols;
    const int h = lane / 16;
    const int nvalid = (int)min((int64_t)NT, a.N);
    const int kpart = wave % P, sub = wave / P;
    const int64_t q0 = qb * kpart / P, q1 = qb * (kpart + 1) / P;
    const int64_t nq = q1 - q0;  // blocks of this wave per tile (may be 0)
    const int64_t total = group_tiles(a);
    const int64_t ngroups = (total + TPW - 1) / TPW;
    const int64_t nit = (ngroups - blockIdx.x + gridDim.x - 1) / gridDim.x;
    // tile of this wave in iteration it (may be >= total in the last one)
    auto tile_of = [&](int64_t it) { return (blockIdx.x + it * gridDim.x) * TPW + sub; };
    const bool has_work = nq > 0 && tile_of(0) < total;
    const int64_t nslots = has_work ? nit * nq : 0;

    // Load cursor: slot li = (iteration lit, block lq); lp points at this
    // lane's 16 bytes of it.  Past the last valid slot the cursor stays put,
    // so every ring load below is unconditional (a harmless reload): with no
    // load behind a branch the compiler keeps exactly RING - 1 loads in
    // flight when it waits for the oldest.
    int64_t li = 0, lit = 0, lq = q0;
    bool lvalid = has_work;  // the cursor is on a slot of a real tile
    gptr<const v4u> lp = nullptr;
    if (has_work) lp = slot_ptr(resolve_tile(a, tile_of(0)), qb, q0, lane);
    auto advance_load = [&]() {
        if (++li >= nslots || !lvalid) return;  // stay on the last valid slot
        if (++lq < q1) {
            lp += kWave;  // next 1 KiB block of the same row tile
            return;
        }
        lq = q0;
        ++lit;
        const int64_t t = tile_of(lit);
        if (t < total) lp = slot_ptr(resolve_tile(a, t), qb, q0, lane);
        else lvalid = false;  // tiles ran out in the last iteration
    };

    // ---- prologue, part 1: global loads of the activations ----
    // They are issued before the first ring fill, so they return first and
    // the activation staging below overlaps the HBM latency of the weights.
    // With the quantization fused (MODE 0) the ring fill waits until after
    // the absmax barrier: issued earlier, it queues with the activation loads
    // and holds up every wave's arrival there (2.3 % on the 70B-class block
    // as four launches).
    constexpr int kUnits = sizeof(Raw8<T>) / 16;
    constexpr int kChunks = kRawUnits / (NT * kUnits);  // MODE 0: raw chunks
    constexpr int kCopy = (int)((kDecLdsMax + 16 * kThreads - 1) / (16 * kThreads));  // MODE 1
    Raw8<T> raw[MODE == 0 ? NT : 1][MODE == 0 ? kChunks : 1];
    v4u cpy[MODE == 1 ? kCopy : 1];
    const T *xin = static_cast<const T *>(dx.x);
    // Every load is unconditional (out-of-range chunks re-read the last valid
    // one and are masked below), again so that no load sits behind a branch.
    if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const int64_t k = min(8 * ((int64_t)threadIdx.x + (int64_t)c * kThreads), K - 8);
                raw[j][c].load(xin + min(j, nvalid - 1) * K + k);
            }
    } else if (MODE == 1) {
        // NT*K <= kDecLdsMax <= kCopy * 16 * kThreads bytes
#pragma unroll
        for (int c = 0; c < kCopy; ++c) {
            const int64_t e = min(16 * ((int64_t)threadIdx.x + (int64_t)c * kThreads),
                                  nvalid * K - 16);
            cpy[c] = *to_global(reinterpret_cast<const v4u *>(dx.xq + e));
        }
    }

    // Weight scales of the group's projections: loaded before the ring fill
    // and written to LDS at the end of the prologue, so that no wait for them
    // also waits for the ring's HBM round trip (the vector-memory counter
    // retires in order).
    float wsc = 0.0f;
    if (threadIdx.x < kMaxGroup) wsc = group_weight_scale(a, threadIdx.x);

    // First ring fill.
    v4u ring[RING];
    auto fill = [&]() {
        if (has_work) {
#pragma unroll
            for (int d = 0; d < RING; ++d) {
                ring[d] = __builtin_nontemporal_load(lp);
                advance_load();
            }
        }
    };
    if (MODE != 0) fill();

    // ---- prologue, part 2: int8 activations of every token into LDS ----
    const int8_t *xsrc;
    if (MODE == 0) {
        float amax[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            uint32_t mb = 0;
#pragma unroll
            for (int c = 0; c < kChunks; ++c)  // re-read chunks cannot change a max
                mb = max(mb, raw[j][c].abs_bits());
            mb = wave_max_u32(mb);
            if (lane == 0) s_amax[wave][j] = mb;
        }
        __syncthreads();
        fill();
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            uint32_t mb = s_amax[0][j];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) mb = max(mb, s_amax[w][j]);
            amax[j] = __uint_as_float(mb);
            const float inv = quant_inv(amax[j]);
            int sum = 0;
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const int64_t k = 8 * ((int64_t)threadIdx.x + (int64_t)c * kThreads);
                int part = 0;
                const uint2 q = quant8(raw[j][c].eight(), inv, part);
                if (j < nvalid && k < K) {
                    *reinterpret_cast<uint2 *>(smem + j * K + k) = q;
                    sum += part;
                }
            }
            sum = wave_sum(sum);
            if (lane == 0) s_sum[wave][j] = sum;
        }
        __syncthreads();
        if (threadIdx.x < NT) {
            const int j = threadIdx.x;
            int t = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) t += s_sum[w][j];
            s_xsum[j] = t;
            s_scale[j] = amax[j];
        }
        xsrc = smem;
    } else if (MODE == 1) {
#pragma unroll
        for (int c = 0; c < kCopy; ++c) {
            const int64_t e = 16 * ((int64_t)threadIdx.x + (int64_t)c * kThreads);
            if (e < nvalid * K) *reinterpret_cast<v4u *>(smem + e) = cpy[c];
        }
        if ((int)threadIdx.x < nvalid) {
            s_xsum[threadIdx.x] = dx.xsum[threadIdx.x];
            s_scale[threadIdx.x] = dx.xs[threadIdx.x];
        }
        xsrc = smem;
    } else {
        if ((int)threadIdx.x < nvalid) {
            s_xsum[threadIdx.x] = dx.xsum[threadIdx.x];
            s_scale[threadIdx.x] = dx.xs[threadIdx.x];
        }
        xsrc = dx.xq;
    }
    if (threadIdx.x < kMaxGroup) s_wscale[threadIdx.x] = wsc;
    __syncthreads();
    // dequantization factor per (projection, token)
    if (threadIdx.x < kMaxGroup * NT) {
        const int p = threadIdx.x / NT, j = threadIdx.x % NT;
        s_factor[p][j] = token_factor(s_wscale[p], s_scale[j]);
    }
    __syncthreads();
    // Rows of tokens >= N are never read (dot_slot stops at nvalid).
    const int8_t *xb = xsrc + 16 * h;

    // ---- tiles ----
    int buf = 0;
    Acc<NT> acc;
    acc_zero(acc);
    // Finish iteration it: reduce this wave's sums and write the outputs of
    // the iteration's tiles.  With P > 1 every wave calls this once per
    // iteration, in order (it holds one barrier).
    auto iter_done = [&](int64_t it) {
        int v[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            v[j] = acc.a1[j] + (acc.a4[j] >> 2) + (acc.a16[j] >> 4);
            v[j] += __shfl_xor(v[j], 16, kWave);
            v[j] += __shfl_xor(v[j], 32, kWave);
        }
        acc_zero(acc);
        if (P == 1) {
            const int64_t tile = tile_of(it);
            if (lane < 16 && tile < total) {
                const TileRef tr = resolve_tile(a, tile);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    if (j >= nvalid) break;
                    store_out(tr.y, a.ydt, j * tr.M + tr.mt * kTileRows + lane, v[j] - s_xsum[j],
                              s_factor[tr.proj][j]);
                }
            }
        } else {
            if (lane < 16) {
#pragma unroll
                for (int j = 0; j < NT; ++j) red[buf][wave][j][lane] = v[j];
            }
            __syncthreads();
            if (threadIdx.x < TPW * 16 * NT) {
                const int s = threadIdx.x / (16 * NT);
                const int j = (threadIdx.x / 16) % NT, r = threadIdx.x % 16;
                const int64_t tile = (blockIdx.x + it * gridDim.x) * TPW + s;
                if (j < nvalid && tile < total) {
                    const TileRef tr = resolve_tile(a, tile);
                    int t = 0;
#pragma unroll
                    for (int p = 0; p < P; ++p) t += red[buf][s * P + p][j][r];
                    store_out(tr.y, a.ydt, j * tr.M + tr.mt * kTileRows + r, t - s_xsum[j],
                              s_factor[tr.proj][j]);
                }
            }
            buf ^= 1;
        }
    };

    if (!has_work) {
        // no slots: still take part in every iteration's reduction
        if (P > 1)
            for (int64_t it = 0; it < nit; ++it) iter_done(it);
        return;
    }
    int64_t cq = q0, cit = 0;  // compute cursor: block, iteration
    for (int64_t base = 0; base < nslots; base += RING) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            const int64_t i = base + d;
            const v4u cur = ring[d];
            ring[d] = __builtin_nontemporal_load(lp);
            advance_load();
            if (i < nslots) {
                dot_slot<NT>(cur, xb + cq * kTileCols, K, nvalid, acc);
                if (++cq == q1) {
                    iter_done(cit);
                    cq = q0;
                    ++cit;
                }
            }
        }
    }
}

int tokens_per_pass(int64_t N) { return N == 1 ? 1 : (N == 2 ? 2 : 4); }

// Whether the fused prologue can hold the raw input of every token.
bool fused_fits(int64_t N, int64_t K, bt_dtype xdt) {
    const int64_t nt = tokens_per_pass(N);
    const int64_t units = xdt == BT_F32 ? 2 : 1;
    const int64_t chunks_needed = (K / 8 + kDecThreads - 1) / kDecThreads;
    return nt * K <= kDecLdsMax && chunks_needed * nt * units <= kRawUnits;
}

template <typename T, int NT, int MODE>
hipError_t launch_dec(const GroupArgs &a, const DecodeX &dx, size_t shmem, hipStream_t s) {
    constexpr int TPW = kDecWaves / kDecSplit;
    const int64_t groups = (group_tiles(a) + TPW - 1) / TPW;
    const int per_cu = shmem <= 48 * 1024 ? kDecPerCu : 1;
    const int64_t grid = min(groups, (int64_t)device_cus() * per_cu);
    hipLaunchKernelGGL((decode_dot4_kernel<T, NT, MODE, kDecWaves, kDecSplit, kRing>),
                       dim3((unsigned)grid), dim3(kDecThreads), shmem, s, a, dx);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_dec_nt(const GroupArgs &a, const DecodeX &dx, int mode, bt_dtype xdt,
                         hipStream_t s) {
    const size_t lds = (size_t)(NT * a.K);
    if (mode == 0)
        return xdt == BT_F32 ? launch_dec<float, NT, 0>(a, dx, lds, s)
                             : launch_dec<uint16_t, NT, 0>(a, dx, lds, s);
    if (mode == 1) return launch_dec<uint16_t, NT, 1>(a, dx, lds, s);
    return launch_dec<uint16_t, NT, 2>(a, dx, 0, s);
}

hipError_t launch_dec_any(const GroupArgs &a, const DecodeX &dx, int mode, bt_dtype xdt,
                          hipStream_t s) {
    if (a.N == 1) return launch_dec_nt<1>(a, dx, mode, xdt, s);
    if (a.N == 2) return launch_dec_nt<2>(a, dx, mode, xdt, s);
    return launch_dec_nt<4>(a, dx, mode, xdt, s);
}

}  // namespace

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

hipError_t launch_mfma_decode(const GroupArgs &a, hipStream_t s);

// From 2 tokens on, the dot4 kernel reads every token's activation words from
// LDS for each weight slot (four 16-byte reads per token per slot), so it
// turns LDS- and ALU-bound where the weight stream is long, while the
// matrix-core kernel costs about the same for any N <= 16 but needs many row
// tiles to fill the chip.  Measured per call (bf16 out, each call on its own
// weight copy): at 2 tokens dot4 is as fast or faster except on the longest
// rows (8192 x 28672: 17.6 vs 16.4 us); at 3-4 tokens it is faster on short
// groups (2560 x 2560 and 2560 x 6912: 5.1-6.7 vs 5.8-7.8 us) and slower on
// tall ones (6912 x 2560 at 3 tokens: 6.5 vs 6.0 us; 8192 x 8192 at 4: 9.6 vs
// 8.2 us); rows whose codes exceed its LDS (NT * K above 64 KiB) make it read
// them from global memory at twice the time (8192 x 28672 at 3 tokens: 35.3
// vs 16.8 us).
bool decode_dot4(int64_t N, int64_t M, int64_t K) {
    if (N < 1 || N > kDot4MaxN) return false;
    if (N == 1) return true;
    if (tokens_per_pass(N) * K > kDecLdsMax) return false;
    return M < 4096 || (N == 2 && K < 16384);
}

hipError_t launch_decode(const Group &g, hipStream_t s) {
    if (g.N == 0) return hipSuccess;
    const GroupArgs a = make_group_args(g);
    if (!decode_dot4(g.N, group_rows(g), g.K)) return launch_mfma_decode(a, s);
    const DecodeX dx{nullptr, g.xq, g.xs, g.xsum};
    const int mode = tokens_per_pass(g.N) * g.K <= kDecLdsMax ? 1 : 2;
    return launch_dec_any(a, dx, mode, BT_BF16, s);
}

bool decode_fuses_quant(int64_t N, int64_t M, int64_t K, bt_dtype xdt) {
    return decode_dot4(N, M, K) && fused_fits(N, K, xdt);
}

hipError_t launch_decode_fused(const Group &g, const void *x, bt_dtype xdt, hipStream_t s) {
    const GroupArgs a = make_group_args(g);
    const DecodeX dx{x, nullptr, nullptr, nullptr};
    return launch_dec_any(a, dx, 0, xdt, s);
}

}  // namespace bt
