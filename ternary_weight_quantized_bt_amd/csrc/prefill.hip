// prefill.hip -- tiled int8 matrix-core product for many tokens (prefill).
//
// The ternary contraction ([PARA] section 5, figure "BitNet b1.58 Ternary
// Matrix Multiplication") is a dense int8 contraction once the codes 0/1/2
// ([I2S] "Ternary Representation and Packing") are unpacked:
//   acc[n,m] = sum_k code[m,k] * xq[n,k] - xsum[n]
// so it runs on v_mfma_i32_16x16x64_i8 with an exact int32 accumulate.
//
// Work decomposition.  A workgroup computes a BM x BN output tile (BM rows of
// the grouped projections, BN tokens) with WMW x WNW waves; a wave owns
// RT row tiles x TG token groups of 16 x 16.  The K loop walks 256-column
// blocks:
//   * A (weights): every lane loads its 16-byte packed slot of each of its RT
//     row tiles straight into registers (T16Q256: word t of the slot is the
//     16 codes of row lane%16, columns 64*t + 16*(lane/16) + 0..15), and one
//     word unpacks with shifts and masks into the lane's A operand of one
//     16x16x64 instruction.  Weights never touch LDS.
//   * B (activations): the BN x 256 int8 block is copied global -> LDS with
//     the direct 16-byte LDS-load instruction (no registers), double
//     buffered, the next block in flight while the current one is consumed.
//     Both loads go through buffer resources (the tile's token rows, each
//     row tile's packed slots): a lane's offset is fixed for the tile and the
//     block's offset is a scalar, so the K loop does no address arithmetic
//     on the vector unit (-2 % per prefill step).
//     Inside a token's 256-byte row, 16-byte chunk c is stored at position
//     c ^ (token % 16), so the 16 lanes that read one chunk of 16 different
//     tokens hit 16 different bank groups.
//   * The accumulators start at minus the token's code sum, so after the
//     last block they hold the exact sum; the epilogue dequantizes it
//     (float32: acc * (s_w * s_a / 127)) to fp32 / bf16, or writes it.
// The tile order is XCD-aware: workgroups are handed to the eight XCDs
// round-robin, so workgroup i is mapped to position (i % 8) * ceil(T / 8) +
// i / 8 of a tile list made of chunks of ceil(ntok / 8) token tiles, each
// chunk walked row tile by row tile (all of the chunk's token tiles of one
// row tile, then the next row tile).  An XCD then works through about one
// chunk: its activation rows stay in its L2, and each weight tile is used by
// the chunk's token tiles back to back, so it is fetched into that L2 once
// rather than once per token tile (-4 % time per prefill step together with
// the epilogue loads hoisted to the tile's start).

#include <algorithm>

#include "group.hpp"

namespace bt {

namespace {

constexpr int kXcds = 8;

// Buffer-resource loads, declared by their LLVM intrinsic names (a plain
// declaration also parses in the compiler's host pass).  A raw buffer load
// reads base + voffset (per lane) + soffset (scalar) and returns zeros past
// num_records bytes; the resource is base, stride 0, num_records and the
// data-format word of gfx9-family raw buffers.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ void bt_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) void *lds, int size,
                                   int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");
__device__ i32x4_t bt_buffer_load_b128(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ __forceinline__ i32x4_t bt_make_rsrc(const void *p, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return i32x4_t{(int)(uint32_t)a, (int)(uint32_t)(a >> 32) & 0xFFFF, bytes, 0x00020000};
}


__device__ __forceinline__ v4i unpack_a(uint32_t word) {
    v4i a;
    a.x = (int)codes_of_group(word, 0);
    a.y = (int)codes_of_group(word, 1);
    a.z = (int)codes_of_group(word, 2);
    a.w = (int)codes_of_group(word, 3);
    return a;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// One group's work; b is the workgroup's number among the G that run the
// group (blockIdx.x and gridDim.x of a launch for this group alone; b is a
// multiple of 8 apart from the launch's own numbering, so the XCD of a
// workgroup is b % 8 either way).
template <int RT, int TG, int WMW, int WNW, int S>
__device__ __forceinline__ void prefill_group(const GroupArgs &a, int64_t mtiles, int64_t b,
                                              int64_t G) {
    constexpr int kWaves = WMW * WNW;
    constexpr int BN = 16 * TG * WNW;       // tokens per workgroup tile
    constexpr int BMT = RT * WMW;           // row tiles per workgroup tile
    constexpr int kRow = kTileCols;         // bytes of one token row of a block
    constexpr int kDma = BN * kRow / 1024;  // 1 KiB direct loads per block
    static_assert(kDma % kWaves == 0, "direct loads must split evenly over the waves");
    constexpr int kDmaW = kDma / kWaves;    // per wave and block
    constexpr int kVm = RT + kDmaW;         // vector-memory operations per wave and block
    static_assert((S - 2) * kVm <= 63, "wait count exceeds the counter");
    // One LDS object per stage (not one array): the compiler can then see that
    // a direct load into one stage does not alias reads of another, and need
    // not drain every outstanding load before each barrier.
    __shared__ __attribute__((aligned(1024))) int8_t sB0[BN * kRow];
    __shared__ __attribute__((aligned(1024))) int8_t sB1[BN * kRow];
    __shared__ __attribute__((aligned(1024))) int8_t sB2[S > 2 ? BN * kRow : 16];
    __shared__ __attribute__((aligned(1024))) int8_t sB3[S > 3 ? BN * kRow : 16];
    static_assert(S >= 2 && S <= 4, "two to four stages");
    auto stage = [&](int st) -> int8_t * {
        return st == 0 ? sB0 : (st == 1 ? sB1 : (st == 2 ? sB2 : sB3));
    };

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WNW, wn = wave % WNW;
    const int r = lane % 16, h = lane / 16;
    const int64_t K = a.K, qb = K / kTileCols, N = a.N;
    const int64_t total = group_tiles(a);  // 16-row tiles of the group

    // XCD-aware tile order (see the header).
    const int64_t ntok = (N + BN - 1) / BN;
    const int64_t ntiles = mtiles * ntok;
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    // The workgroup takes list positions b, b + G, b + 2G, ... (G is a
    // multiple of 8, so they all belong to its own XCD's run).  A launch for
    // one group caps G at the resident workgroups, so the grid is persistent
    // and one tile's stores drain while the next computes; the four-group
    // launch gives every position its own workgroup.
    for (int64_t j = b;; j += G) {
        const int64_t idx = (j % kXcds) * per_xcd + j / kXcds;
        if (j / kXcds >= per_xcd || idx >= ntiles) break;  // whole workgroup
        // chunk cc of TCH token tiles (the last may be shorter), row tile
        // major within it
        const int64_t TCH = (ntok + kXcds - 1) / kXcds;
        const int64_t chunk = mtiles * TCH;
        const int64_t cc = idx / chunk, rr = idx - cc * chunk;
        const int64_t tcn = min(TCH, ntok - cc * TCH);
        const int64_t tm = rr / tcn, tn = cc * TCH + rr % tcn;
        const int64_t tok0 = tn * BN;

        // This wave's row tiles (clamped to the last tile past the end; their
        // results are not stored): wave-uniform base addresses plus the lane's
        // 16-byte offset at each load.
        const uint8_t *abase[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const TileRef tr = resolve_tile(a, min(tm * BMT + wm * RT + i, total - 1));
            abase[i] = tr.packed + tr.mt * qb * kTileBytes;
        }

        // All loads of block q (clamped to the last block, so every call issues
        // exactly kVm operations and the wait counts below stay exact): the A
        // slots into registers, the token block into LDS stage st.  Each 1 KiB
        // direct load covers 4 tokens; lane l fills position l%16 of token l/16
        // with global chunk (l%16) ^ (token % 16).
        v4u ar[S][RT];
        // The tile's token rows as one buffer resource (its rows only: at most
        // BN * K < 2^32 bytes), so each direct load is a 32-bit lane offset
        // fixed for the tile plus the block's column offset in a scalar.
        const i32x4_t xrs = bt_make_rsrc(a.xq + tok0 * K, (int)(min((int64_t)BN, N - tok0) * K));
        i32x4_t ars[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) ars[i] = bt_make_rsrc(abase[i], (int)(qb * kTileBytes));
        int dvoff[kDmaW];
#pragma unroll
        for (int i = 0; i < kDmaW; ++i) {
            const int d = wave * kDmaW + i;   // 1 KiB unit of the block
            const int tl = d * 4 + lane / 16;  // token within the tile
            const int64_t tok = min(tok0 + tl, N - 1);
            const int c = (lane % 16) ^ (tl % 16);
            dvoff[i] = (int)((tok - tok0) * K + 16 * c);
        }
        auto issue = [&](int64_t q, int st) {
            q = min(q, qb - 1);
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const i32x4_t v = bt_buffer_load_b128(ars[i], 16 * lane, (int)(q * kTileBytes), 0);
                ar[st][i] = v4u{(unsigned)v.x, (unsigned)v.y, (unsigned)v.z, (unsigned)v.w};
            }
#pragma unroll
            for (int i = 0; i < kDmaW; ++i) {
                const int d = wave * kDmaW + i;
                bt_buffer_load_lds(
                    xrs, (__attribute__((address_space(3))) void *)(stage(st) + d * 1024), 16,
                    dvoff[i], (int)(q * kTileCols), 0, 0);
            }
        };
        // B fragment of token group g, 64-column step t, from stage st: token
        // g*16 + r of this wave, chunk 4t + h, stored at (4t + h) ^ (token % 16).
        auto read_b = [&](int st, int t, int g) {
            return *reinterpret_cast<const v4i *>(stage(st) + (wn * 16 * TG + g * 16 + r) * kRow +
                                                  16 * ((4 * t + h) ^ r));
        };

        // The epilogue's per-token and per-tile factors, loaded now so their
        // latency hides under the K loop.
        float xs_pre[TG];
        int32_t xsum_pre[TG];
#pragma unroll
        for (int g = 0; g < TG; ++g) {
            const int64_t tc = min(tok0 + wn * 16 * TG + g * 16 + r, N - 1);
            xs_pre[g] = a.xs[tc];
            xsum_pre[g] = a.xsum[tc];
        }
        float s_w[RT];
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const TileRef tr = resolve_tile(a, min(tm * BMT + wm * RT + i, total - 1));
            s_w[i] = packed_scale(tr.packed, tr.M, K);
        }

        // Accumulators start at minus the token's code sum, so they end at
        // sum (code - 1) * xq (exact in int32) with no subtraction after.
        v4i acc[RT][TG];
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int g = 0; g < TG; ++g)
                acc[i][g] = v4i{-xsum_pre[g], -xsum_pre[g], -xsum_pre[g], -xsum_pre[g]};

        // Prologue: blocks 0 .. S-2 in flight.
#pragma unroll
        for (int s = 0; s < S - 1; ++s) issue(s, s);

        // Block q: wait until it has landed for every wave (S-2 younger blocks
        // may stay in flight), barrier -- which also means every wave is done
        // with block q-1 -- then refill that block's stage with block q+S-1 and
        // compute block q.  Unrolled by S so stages and registers are static.
        for (int64_t q0 = 0; q0 < qb; q0 += S) {
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int64_t q = q0 + s;
                if (q >= qb) break;  // uniform
                // Block q's direct loads are complete for this wave once at most
                // the S-2 younger blocks are outstanding; the bare barrier (no
                // fence: a fence would drain those younger loads too) then makes
                // every wave's part of the block visible.
                __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * kVm));
                __builtin_amdgcn_s_barrier();
                // (two stages: the wait above is for zero operations, so the
                // clamped reload past the last block can be left out)
                if (S > 2 || q + 1 < qb) issue(q + S - 1, (s + S - 1) % S);
                v4i bcur[TG], bnext[TG];
#pragma unroll
                for (int g = 0; g < TG; ++g) bcur[g] = read_b(s, 0, g);
                v4i A[RT];
#pragma unroll
                for (int i = 0; i < RT; ++i) A[i] = unpack_a(ar[s][i][0]);
                // The next step's fragments are read while this step's matrix
                // instructions run; a scheduling fence per step keeps the
                // scheduler from hoisting every step's operands at once.
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (t < 3) {
#pragma unroll
                        for (int g = 0; g < TG; ++g) bnext[g] = read_b(s, t + 1, g);
                    }
                    // next step's A operands, unpacked between this step's
                    // matrix instructions (one instruction, two VALU ops)
                    v4i An[RT];
                    if (t < 3) {
#pragma unroll
                        for (int i = 0; i < RT; ++i) An[i] = unpack_a(ar[s][i][t + 1]);
                    }
#pragma unroll
                    for (int g = 0; g < TG; ++g)
#pragma unroll
                        for (int i = 0; i < RT; ++i)
                            acc[i][g] =
                                __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i], bcur[g], acc[i][g], 0, 0, 0);
                    if (t < 3) {
#pragma unroll
                        for (int g = 0; g < TG; ++g) bcur[g] = bnext[g];
#pragma unroll
                        for (int i = 0; i < RT; ++i) A[i] = An[i];
                    }
#pragma unroll
                    for (int k = 0; k < RT * TG; ++k) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
                    }
                }
            }
        }

        // Epilogue: lane (r, h) holds rows 4h..4h+3 of each row tile for token
        // g*16 + r of each group.  Per-row-tile values are wave-uniform; token
        // values are loaded from a clamped index so only the stores branch.
        // bf16 output with all of the workgroup's row tiles in one projection
        // (every tile but those at a projection boundary or past the end): the
        // results of 16 tokens at a time go through LDS, token-major, and each
        // token's BMT*16 consecutive outputs leave with 16-byte stores that
        // cover whole rows (a lane's own 4 outputs per token would be 8-byte
        // pieces 2*M bytes apart).  The B stages are free by then; sB0 and sB1
        // alternate, so one barrier per token group orders the writes of one
        // group and the reads of the previous one.
        bool stored = false;
        if constexpr (WNW == 1) {
            const int64_t wt0 = tm * BMT;
            bool whole = false;
            TileRef tw{};
            if (a.ydt == BT_BF16 && wt0 + BMT - 1 < total) {
                tw = resolve_tile(a, wt0);
                whole = resolve_tile(a, wt0 + BMT - 1).proj == tw.proj;
            }
            if (whole) {
                constexpr int kRowsWg = BMT * kTileRows;     // outputs per token
                constexpr int kPitch = 2 * kRowsWg + 16;     // LDS bytes per token (padded)
                constexpr int kPerTok = 2 * kRowsWg / 16;    // 16-byte chunks per token
                static_assert(16 * kPitch <= BN * kRow, "16 tokens fit one stage");
                // row tiles of one projection share its scale
                const float sw = s_w[0];
                __syncthreads();  // every wave is done with the B stages (and their loads)
#pragma unroll
                for (int g = 0; g < TG; ++g) {
                    int8_t *T = (g & 1) ? sB1 : sB0;
                    const float f = token_factor(sw, xs_pre[g]);
#pragma unroll
                    for (int i = 0; i < RT; ++i) {
                        const v4i v = acc[i][g];
                        typedef unsigned v2u __attribute__((ext_vector_type(2)));
                        *reinterpret_cast<v2u *>(T + r * kPitch + 2 * ((wm * RT + i) * kTileRows + 4 * h)) =
                            v2u{f32x2_to_bf16x2(__fmul_rn((float)v.x, f), __fmul_rn((float)v.y, f)),
                                f32x2_to_bf16x2(__fmul_rn((float)v.z, f), __fmul_rn((float)v.w, f))};
                    }
                    __syncthreads();
                    for (int c = (int)threadIdx.x; c < 16 * kPerTok; c += kWaves * kWave) {
                        const int tl = c / kPerTok, col = c % kPerTok;
                        const int64_t tok = tok0 + g * 16 + tl;
                        if (tok < N)  // written once: non-temporal
                            __builtin_nontemporal_store(
                                *reinterpret_cast<const v4u *>(T + tl * kPitch + 16 * col),
                                to_global(reinterpret_cast<v4u *>(reinterpret_cast<uint16_t *>(tw.y) +
                                                                  tok * tw.M + tw.mt * kTileRows) + col));
                    }
                }
                stored = true;
            }
        }

        if (!stored) {
#pragma unroll
            for (int g = 0; g < TG; ++g) {
                const int64_t tok = tok0 + wn * 16 * TG + g * 16 + r;
                const float s_a = xs_pre[g];
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    const int64_t t = tm * BMT + wm * RT + i;
                    if (t >= total) continue;  // uniform
                    const TileRef tr = resolve_tile(a, t);
                    const float f = token_factor(s_w[i], s_a);
                    const int64_t base = tok * tr.M + tr.mt * kTileRows + 4 * h;
                    if (tok < N) store_out4(tr.y, a.ydt, base, acc[i][g], 0, f);
                }
                __builtin_amdgcn_sched_barrier(0);  // keep one token group's values live at a time
            }
        }
        // every wave is done with the stages (and their loads) before the next
        // tile's first loads go into them
        __syncthreads();
    }
}

template <int RT, int TG, int WMW, int WNW, int S>
__global__ __launch_bounds__(WMW * WNW * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(GroupArgs a, int64_t mtiles) {
    prefill_group<RT, TG, WMW, WNW, S>(a, mtiles, blockIdx.x, gridDim.x);
}

// Up to four groups (each with its own input) in one grid: workgroups
// [start[i], start[i+1]) run group i; every range is a multiple of 8 long.
constexpr int kMaxMulti = 4;
struct MultiArgs {
    GroupArgs g[kMaxMulti];
    int64_t mtiles[kMaxMulti];
    int start[kMaxMulti + 1];
};

template <int RT, int TG, int WMW, int WNW, int S>
__global__ __launch_bounds__(WMW * WNW * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_multi_kernel(MultiArgs m) {
    const int b = (int)blockIdx.x;
    if (b < m.start[1])
        prefill_group<RT, TG, WMW, WNW, S>(m.g[0], m.mtiles[0], b, m.start[1]);
    else if (b < m.start[2])
        prefill_group<RT, TG, WMW, WNW, S>(m.g[1], m.mtiles[1], b - m.start[1], m.start[2] - m.start[1]);
    else if (b < m.start[3])
        prefill_group<RT, TG, WMW, WNW, S>(m.g[2], m.mtiles[2], b - m.start[2], m.start[3] - m.start[2]);
    else
        prefill_group<RT, TG, WMW, WNW, S>(m.g[3], m.mtiles[3], b - m.start[3], m.start[4] - m.start[3]);
}

// Workgroups of one group: its tiles, rounded up to a multiple of the XCDs.
template <int RT, int TG, int WMW, int WNW>
int64_t group_grid(const GroupArgs &a, int64_t &mtiles) {
    constexpr int BMT = RT * WMW, BN = 16 * TG * WNW;
    mtiles = (group_tiles(a) + BMT - 1) / BMT;
    const int64_t ntiles = mtiles * ((a.N + BN - 1) / BN);
    return (ntiles + kXcds - 1) / kXcds * kXcds;
}

// Resident workgroups of a persistent grid: two per CU (registers), a
// multiple of the XCD count.
inline int64_t prefill_slots() { return max((int64_t)kXcds, (int64_t)device_cus() * 2 / kXcds * kXcds); }

template <int RT, int TG, int WMW, int WNW, int S>
hipError_t launch_multi(const GroupArgs *gs, int count, hipStream_t s) {
    // One workgroup per tile here (not persistent): the hardware hands the
    // next workgroup to whichever slot frees up, which balances the groups'
    // different tile costs better than any static split of the slots
    // (measured).  Largest K first, so the cheap tiles fill the tail.
    int order[kMaxMulti];
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order, order + count, [&](int x, int y) { return gs[x].K > gs[y].K; });
    MultiArgs m{};
    int64_t start = 0;
    for (int i = 0; i < kMaxMulti; ++i) {
        const int j = order[i < count ? i : count - 1];
        m.g[i] = gs[j];
        m.start[i] = (int)start;
        const int64_t grid = group_grid<RT, TG, WMW, WNW>(gs[j], m.mtiles[i]);
        if (i < count) start += grid;
        if (start > INT32_MAX) return hipErrorInvalidConfiguration;  // grid.x limit
    }
    m.start[kMaxMulti] = (int)start;
    if (start == 0) return hipSuccess;
    hipLaunchKernelGGL((prefill_multi_kernel<RT, TG, WMW, WNW, S>), dim3((unsigned)start),
                       dim3(WMW * WNW * kWave), 0, s, m);
    return hipGetLastError();
}

template <int RT, int TG, int WMW, int WNW, int S>
hipError_t launch_tiles(const GroupArgs &a, hipStream_t s) {
    int64_t mtiles;
    const int64_t grid = min(group_grid<RT, TG, WMW, WNW>(a, mtiles), prefill_slots());
    hipLaunchKernelGGL((prefill_kernel<RT, TG, WMW, WNW, S>), dim3((unsigned)grid),
                       dim3(WMW * WNW * kWave), 0, s, a, mtiles);
    return hipGetLastError();
}

}  // namespace

// 256 rows x 64 tokens per workgroup (4 waves of 64 x 64), two stages of
// 16 KiB (the next block in flight while one is consumed; a third stage
// measured slower -- it costs 16 more registers per lane): two workgroups
// per CU.
hipError_t launch_prefill(const Group &g, hipStream_t s) {
    if (g.N == 0) return hipSuccess;
    const GroupArgs a = make_group_args(g);
    return launch_tiles<4, 4, 4, 1, 2>(a, s);
}

hipError_t launch_prefill_groups(const Group *groups, int count, hipStream_t s) {
    if (count < 1 || count > kMaxMulti) return hipErrorInvalidValue;
    if (groups[0].N == 0) return hipSuccess;
    GroupArgs gs[kMaxMulti];
    for (int i = 0; i < count; ++i) gs[i] = make_group_args(groups[i]);
    return launch_multi<4, 4, 4, 1, 2>(gs, count, s);
}

}  // namespace bt
