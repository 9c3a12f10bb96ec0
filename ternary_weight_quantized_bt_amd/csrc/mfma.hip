// mfma.hip -- batched decode: a few to a hundred tokens per weight pass, on
// the int8 matrix cores.
//
// The ternary contraction ([PARA] section 5, figure "BitNet b1.58 Ternary
// Matrix Multiplication") is a dense int8 contraction once the codes
// 0/1/2 ([I2S] "Ternary Representation and Packing") are unpacked, so each
// 64-column step runs on one v_mfma_i32_16x16x64_i8 (16 rows x 16 tokens):
// acc = sum code*xq, minus the token's code sum at the end.  The weights are
// unpacked once per fragment and reused by all 16 tokens of the instruction
// (the GPU form of the pages' activation-parallel kernel, [I2S] "How I2_S
// Kernels Process the Format").
//
// Operand mapping.  A 16-byte packed slot of lane l holds, in word t, the
// codes of row l%16 at columns 64*t + 16*(l/16) + 0..15; unpacking one word
// gives exactly the 16 int8 A-operand bytes that lane contributes to a
// 16x16x64 instruction over the 64 columns 64*t..64*t+63.  The B operand of
// lane l is the 16 int8 activations of token l%16 at the same 16 columns.
// Because A and B of a lane then cover the same columns in the same byte
// order, the instruction sums over exactly those 64 columns whatever order
// the hardware gives the lane groups.  The 16x16 result lands as: lane l,
// register v = row 4*(l/16) + v, token l%16 -- four consecutive outputs of
// one token, stored with one vector store.
//
// Schedule (the weight stream is the bound: 8 bytes of weights per 4x16
// multiply-adds).  Persistent grid, one 16-token group per workgroup
// (gridDim.y groups for more tokens).  The workgroup stages its tokens' codes
// once, global -> LDS with direct 16-byte loads, and then walks the 16-row
// tiles of the group with a stride of the grid size; within a tile its waves
// split K into contiguous runs of 256-column blocks, and each wave keeps RING
// non-temporal weight-slot loads in flight, running straight across tile
// boundaries (the same ring as the single-token kernel).  In LDS, 16-byte chunk c of token n
// sits at position c ^ (n % 16) of its 256-column block, so the 16 tokens an
// instruction reads fall on 16 different bank groups.  Rows too long for LDS
// are done in K phases: the codes of one K range at a time, all of the
// workgroup's tiles over that range, int32 partial sums kept in LDS between
// phases (exact: the sum is split, not rounded).  Partial sums of the waves
// of a tile meet in LDS (double-buffered, one barrier per tile) and the
// tile's first wave adds them, dequantizes and stores.

#include "group.hpp"

namespace bt {

namespace {

// Launch shape: 16 waves per workgroup, a tile's K split over 4 of them
// (four tiles per iteration), 3 slot loads in flight per wave.  At 8 tokens
// of the 70B-class block this is 6 % faster than 8 waves with a 4-way split
// and 9 % faster than 8 waves with an 8-way split; 12 waves, 2- or 8-way
// splits were slower or equal.  With non-temporal weight loads a ring of 3
// slots per wave is the fastest at 8 tokens (2 / 3 / 4 / 5: 3.62 / 3.56 /
// 3.65 / 3.74 ms per 80 blocks in alternating runs).
constexpr int kMfWaves = 16;
constexpr int kMfThreads = kMfWaves * kWave;
constexpr int kMfSplit = 4;
constexpr int kMfRing = 3;
// LDS of one compute unit and the part a workgroup may use for token codes.
constexpr int64_t kLdsPerCu = 160 * 1024;
constexpr int64_t kMfCodesMax = 128 * 1024;
// With more than one K phase, iterations per workgroup whose partial sums
// stay in LDS (1 KiB each).
constexpr int64_t kMfPhaseTiles = 8;

__device__ __forceinline__ v4i unpack_a(uint32_t word) {
    v4i a;
    a.x = (int)codes_of_group(word, 0);
    a.y = (int)codes_of_group(word, 1);
    a.z = (int)codes_of_group(word, 2);
    a.w = (int)codes_of_group(word, 3);
    return a;
}

// s_waitcnt immediate: at most n vector-memory operations outstanding and no
// LDS operation (expcnt left at its maximum).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

// The workgroup's K range is cut into nph phases of qph 256-column blocks
// (the last may be shorter).  One phase's token codes sit in LDS at a time
// (rows nb * 256 bytes apart); when there is more than one phase, per-tile
// int32 partial sums carry over in LDS, after the codes, from one phase to
// the next, and the last phase dequantizes and stores.
// One group's work; the workgroup is number bx of the gx that run this group
// (blockIdx.x and gridDim.x of a launch for this group alone).
// TL: the weight slots are read with ordinary (cached) loads instead of
// non-temporal ones.
template <int WAVES, int P, int RING, bool TL = false>
__device__ __forceinline__ void mfma_group(const GroupArgs &a, int nph, int qph, int64_t bx,
                                           int64_t gx) {
    static_assert(WAVES % P == 0, "K split must divide the waves");
    constexpr int TPW = WAVES / P;  // tiles per workgroup iteration
    static_assert(RING <= 63, "wait count exceeds the counter");
    extern __shared__ __attribute__((aligned(1024))) int8_t smem[];  // codes, then partials
    __shared__ v4i red[2][TPW][P > 1 ? P - 1 : 1][kWave];
    __shared__ __attribute__((aligned(256))) uint32_t s_tab[kWave];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t K = a.K, qb = K / kTileCols;
    const int r = lane % 16, h = lane / 16;
    const int64_t n0 = 16 * (int64_t)blockIdx.y;        // first token of the workgroup
    const int nrows = (int)min((int64_t)16, a.N - n0);  // its tokens, >= 1
    // B row of this lane.  Result columns of tokens >= nrows depend only on
    // their own (clamped) B rows and are never stored.
    const int rr = min(r, nrows - 1);
    const int kpart = wave % P, sub = wave / P;
    const int64_t total = group_tiles(a);
    const int64_t ngroups = (total + TPW - 1) / TPW;
    const int64_t nit = (ngroups - bx + gx - 1) / gx;
    auto tile_of = [&](int64_t it) { return (bx + it * gx) * TPW + sub; };
    // partial sums: after the codes of the largest phase (16-row allocation)
    const int64_t rows_alloc = min((int64_t)16, a.N);
    v4i *const part = reinterpret_cast<v4i *>(
        smem + ((rows_alloc * qph * kTileCols + 1023) & ~(int64_t)1023));

    // ---- per-token tables ----
    // Per-token code sums and activation scales and the weight scales go to
    // LDS by direct 4-byte loads (no register waits): lane l of every wave
    // fills s_tab[l] -- [0,16) code sums, [16,32) scales (clamped tokens),
    // [32,64) weight scale of projection min(l - 32, 2).
    {
        const uint8_t *src;
        if (lane < 32) {
            const int j = min(lane % 16, nrows - 1);
            src = lane < 16 ? reinterpret_cast<const uint8_t *>(a.xsum + n0 + j)
                            : reinterpret_cast<const uint8_t *>(a.xs + n0 + j);
        } else {
            const int p = min(lane - 32, kMaxGroup - 1);
            const uint64_t m1 = p >= 1 ? ~0ull : 0ull, m2 = p >= 2 ? ~0ull : 0ull;
            const uint8_t *pk = reinterpret_cast<const uint8_t *>(
                pick3(m1, m2, (uint64_t)a.packed[0], (uint64_t)a.packed[1], (uint64_t)a.packed[2]));
            const int64_t M = (int64_t)pick3(m1, m2, (uint64_t)a.M[0], (uint64_t)a.M[1],
                                             (uint64_t)a.M[2]);
            src = pk + M * K / 4;
        }
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)s_tab, 4, 0, 0);
    }

    auto slot_base = [&](int64_t t) {
        const TileRef tr = resolve_tile(a, t);
        return to_global(reinterpret_cast<const v4u *>(tr.packed + tr.mt * qb * kTileBytes)) + lane;
    };

    for (int ph = 0; ph < nph; ++ph) {
        const int64_t kb0 = (int64_t)ph * qph;              // first block of the phase
        const int64_t nb = min((int64_t)qph, qb - kb0);     // its blocks
        const int64_t q0 = kb0 + nb * kpart / P, q1 = kb0 + nb * (kpart + 1) / P;
        const int64_t nq = q1 - q0;  // blocks of this wave per tile (may be 0)
        const bool has_work = nq > 0 && tile_of(0) < total;
        const int64_t nslots = has_work ? nit * nq : 0;
        const bool last = ph == nph - 1;

        if (ph > 0) __syncthreads();  // every wave is done with the previous codes
        // Direct loads of the phase's token codes into LDS.  LDS chunk p (16
        // bytes) = token p / (nb*16), position c = p % (nb*16) of its row; it
        // holds the row's chunk (block kb0 + c/16, within-block chunk
        // (c % 16) ^ (token % 16)).  Lane l of a 1 KiB unit u fills chunk
        // 64u + l; units past the rows (allocation rounded up to 1 KiB)
        // re-read the last chunk.
        {
            const int64_t cpr = nb * 16;
            const int64_t chunks = nrows * cpr;
            const int64_t units = (chunks + 63) / 64;
            for (int64_t u = wave; u < units; u += WAVES) {
                const int64_t p = min(64 * u + lane, chunks - 1);
                const int64_t n = p / cpr, c = p - n * cpr;
                const int8_t *src = a.xq + (n0 + n) * K + kb0 * kTileCols + 16 * (c ^ (n & 15));
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)src,
                    (__attribute__((address_space(3))) void *)(smem + u * 1024), 16, 0, 0);
            }
        }

        // Load cursor (as in the single-token kernel): slot li = (iteration
        // lit, block lq); past the last valid slot it stays put, so every
        // ring load is unconditional and the compiler's wait counts stay
        // exact.  A wave without work points at a valid slot too.
        int64_t li = 0, lit = 0, lq = q0;
        bool lvalid = has_work;
        gptr<const v4u> lp = slot_base(has_work ? tile_of(0) : 0) + (has_work ? q0 : 0) * kWave;
        auto advance_load = [&]() {
            if (++li >= nslots || !lvalid) return;
            if (++lq < q1) {
                lp += kWave;
                return;
            }
            lq = q0;
            ++lit;
            const int64_t t = tile_of(lit);
            if (t < total) lp = slot_base(t) + q0 * kWave;
            else lvalid = false;
        };

        // RING + 1 entries, RING of them in flight: the loop below consumes
        // entry d and then refills entry d - 1, so no entry is live twice and
        // the ring needs no register copies.
        constexpr int kSlots = RING + 1;
        v4u ring[kSlots];
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            ring[d] = (TL ? *lp : __builtin_nontemporal_load(lp));
            advance_load();
        }
        // Everything but the ring is complete and visible after this.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(RING));
        __builtin_amdgcn_s_barrier();

        // LDS byte offsets of this lane's B fragments at the phase's block 0.
        int boff[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) boff[t] = (int)(rr * nb * kTileCols + 16 * ((4 * t + h) ^ rr));

        v4i acc = v4i{0, 0, 0, 0};
        int buf = 0;
        // Finish iteration it: the waves of each tile meet in LDS; the tile's
        // first wave adds the parts (and the earlier phases' partial sum),
        // then keeps the result for the next phase or dequantizes and
        // stores.  Every wave calls this once per iteration, in order (it
        // holds one barrier when P > 1).
        auto iter_done = [&](int64_t it) {
            v4i sum = acc;
            if (P > 1) {
                if (kpart > 0) red[buf][sub][kpart - 1][lane] = acc;
                __syncthreads();
                if (kpart == 0) {
#pragma unroll
                    for (int p = 0; p < P - 1; ++p) sum += red[buf][sub][p][lane];
                }
                buf ^= 1;
            }
            acc = v4i{0, 0, 0, 0};
            const int64_t tile = tile_of(it);
            if (kpart == 0 && tile < total) {
                v4i &keep = part[(it * TPW + sub) * kWave + lane];
                if (ph > 0) sum += keep;
                if (!last) {
                    keep = sum;
                } else if (r < nrows) {
                    const TileRef tr = resolve_tile(a, tile);
                    const float f = token_factor(__uint_as_float(s_tab[32 + tr.proj]),
                                                 __uint_as_float(s_tab[16 + r]));
                    store_out4(tr.y, a.ydt, (n0 + r) * tr.M + tr.mt * kTileRows + 4 * h, sum,
                               (int32_t)s_tab[r], f);
                }
            }
        };

        if (!has_work) {
            for (int64_t it = 0; it < nit; ++it) iter_done(it);
            continue;
        }
        int64_t cq = q0, cit = 0;  // compute cursor: block, iteration
        for (int64_t base = 0; base < nslots; base += kSlots) {
#pragma unroll
            for (int d = 0; d < kSlots; ++d) {
                const int64_t i = base + d;
                if (i < nslots) {
                    const uint32_t words[4] = {ring[d].x, ring[d].y, ring[d].z, ring[d].w};
                    const int8_t *bq = smem + (cq - kb0) * kTileCols;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const v4i B = *reinterpret_cast<const v4i *>(bq + boff[t]);
                        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack_a(words[t]), B, acc, 0, 0, 0);
                    }
                }
                ring[(d + RING) % kSlots] = (TL ? *lp : __builtin_nontemporal_load(lp));
                advance_load();
                if (i < nslots && ++cq == q1) {
                    iter_done(cit);
                    cq = q0;
                    ++cit;
                }
            }
        }
    }
}

template <int WAVES, int P, int RING>
__global__ __launch_bounds__(WAVES * kWave)
void decode_mfma_kernel(GroupArgs a, int nph, int qph) {
    mfma_group<WAVES, P, RING>(a, nph, qph, blockIdx.x, gridDim.x);
}

// Up to four groups (a block's q/k/v, o, gate/up and down, each with its own
// input) in one grid: workgroups [start[i], start[i+1]) run group i.  Each
// branch is the whole single-group body on a fixed argument block, so
// nothing is indexed dynamically.
constexpr int kMaxMulti = 4;
struct MultiArgs {
    GroupArgs g[kMaxMulti];
    int nph[kMaxMulti], qph[kMaxMulti];
    int start[kMaxMulti + 1];  // unused groups have empty ranges
};

template <int WAVES, int P, int RING, bool TL = false>
__global__ __launch_bounds__(WAVES * kWave)
void decode_mfma_multi_kernel(MultiArgs m) {
    const int b = (int)blockIdx.x;
    if (b < m.start[1])
        mfma_group<WAVES, P, RING, TL>(m.g[0], m.nph[0], m.qph[0], b, m.start[1]);
    else if (b < m.start[2])
        mfma_group<WAVES, P, RING, TL>(m.g[1], m.nph[1], m.qph[1], b - m.start[1], m.start[2] - m.start[1]);
    else if (b < m.start[3])
        mfma_group<WAVES, P, RING, TL>(m.g[2], m.nph[2], m.qph[2], b - m.start[2], m.start[3] - m.start[2]);
    else
        mfma_group<WAVES, P, RING, TL>(m.g[3], m.nph[3], m.qph[3], b - m.start[3], m.start[4] - m.start[3]);
}

// Static LDS of a kernel as compiled (the partial-sum buffers and the token
// table), read once per kernel: the dynamic part must fit beside it.
template <typename Kern>
int64_t static_lds(Kern kern) {
    hipFuncAttributes attr{};
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kern)) != hipSuccess) return -1;
    return (int64_t)attr.sharedSizeBytes;
}

hipError_t launch_mf(const GroupArgs &a, int nph, int qph, int64_t grid, size_t shmem,
                     hipStream_t s) {
    auto kern = decode_mfma_kernel<kMfWaves, kMfSplit, kMfRing>;
    if (shmem > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)shmem);
        if (e != hipSuccess) return e;
    }
    const int64_t tgroups = (a.N + 15) / 16;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid, (unsigned)tgroups), dim3(kMfThreads), shmem, s,
                       a, nph, qph);
    return hipGetLastError();
}

// K phases of a group: as few as keep one phase's codes within `cap` bytes.
struct Plan {
    int64_t nph, qph, codes, groups;
};
Plan plan_group(const GroupArgs &a, int64_t cap = kMfCodesMax) {
    constexpr int TPW = kMfWaves / kMfSplit;
    Plan p;
    const int64_t rows = min((int64_t)16, a.N);
    const int64_t qb = a.K / kTileCols;
    const int64_t per_block = rows * kTileCols;
    const int64_t max_blocks = max((int64_t)1, cap / per_block);
    p.nph = (qb + max_blocks - 1) / max_blocks;
    p.qph = (qb + p.nph - 1) / p.nph;
    p.codes = (rows * p.qph * kTileCols + 1023) / 1024 * 1024;
    p.groups = (group_tiles(a) + TPW - 1) / TPW;
    return p;
}

// Partial sums of one iteration's tiles (1 KiB per tile) with more than one
// phase; a workgroup keeps those of each of its iterations.
constexpr int64_t kMfIterPartial = (kMfWaves / kMfSplit) * kWave * 16;

int64_t partial_bytes(const Plan &p, int64_t grid) {
    if (p.nph <= 1) return 0;
    return (p.groups + grid - 1) / grid * kMfIterPartial;
}

// Makes the group's codes plus partial sums fit `avail` bytes of dynamic LDS
// with a grid of at least `grid` workgroups.  With more than one phase a
// workgroup keeps the partial sums of at most kMfPhaseTiles iterations, and
// of fewer when the codes leave less room (the grid grows instead); when not
// even one iteration's partial sums fit beside the codes, the phases get
// shorter.  Returns false if no plan fits.
bool fit_plan(const GroupArgs &a, Plan &p, int64_t &grid, int64_t avail) {
    for (int64_t cap = kMfCodesMax; cap >= (int64_t)kTileCols; cap -= 16 * 1024) {
        Plan q = plan_group(a, cap);
        if (q.nph <= 1) {
            if (q.codes > avail) continue;
            p = q;
            return true;
        }
        const int64_t its = min(kMfPhaseTiles, (avail - q.codes) / kMfIterPartial);
        if (its < 1) continue;
        p = q;
        grid = min(max(grid, (p.groups + its - 1) / its), p.groups);
        return true;
    }
    return false;
}

// The grid of a four-group launch split over the groups (they run side by
// side and should end together): shares in proportion to each group's weight
// bytes, rounded by largest remainders so that they add up to `budget` (the
// workgroups resident at once; one more would wait for a free unit and end a
// whole workgroup's time late), at most one workgroup per tile group.  With
// a single 16-token group, a group that runs in K phases counts 1.3 times
// its bytes: each phase restages the codes and refills the weight ring, and
// the 70B-class down projection (two phases at 8 tokens) then ends closer to
// the others.  Measured against equal weighting in alternating runs: 8 70B-
// class blocks at 8 tokens 0.3544 vs 0.3598 ms (1.1 / 1.2 / 1.3 / 1.4 / 1.6
// in another sweep: 1.2 / 1.8 / 2.3 / -0.4 / -0.5 % faster), a 7B-class block
// at 16 tokens 16 % faster, 70B-class at 2 tokens, 13B- and 34B-class at 8-16
// tokens equal or up to 0.3 % faster; with more token groups it helped some
// shapes and cost others up to 6 %, so it is left out there.
void split_grid(const Plan *p, const int64_t *bytes, int count, int64_t budget, int64_t tgroups,
                int64_t *share) {
    double w[kMaxMulti], rem[kMaxMulti], wsum = 0;
    for (int i = 0; i < count; ++i) {
        w[i] = (double)bytes[i] * (tgroups == 1 && p[i].nph > 1 ? 1.3 : 1.0);
        wsum += w[i];
    }
    int64_t used = 0;
    for (int i = 0; i < count; ++i) {
        const double q = (double)budget * w[i] / wsum;
        share[i] = max((int64_t)1, min(p[i].groups, (int64_t)q));
        rem[i] = q - (double)(int64_t)q;
        used += share[i];
    }
    while (used < budget) {
        int best = -1;
        for (int i = 0; i < count; ++i)
            if (rem[i] >= 0 && share[i] < p[i].groups && (best < 0 || rem[i] > rem[best])) best = i;
        if (best < 0) break;
        ++share[best];
        rem[best] = -1;
        ++used;
    }
}

}  // namespace

hipError_t launch_mfma_decode(const GroupArgs &a, hipStream_t s) {
    if (a.N <= 0 || group_tiles(a) == 0) return hipSuccess;
    if (a.N > kDecodeMaxN) return hipErrorInvalidConfiguration;  // grid y
    static const int64_t stat = static_lds(decode_mfma_kernel<kMfWaves, kMfSplit, kMfRing>);
    if (stat < 0) return hipErrorInvalidDeviceFunction;
    Plan p = plan_group(a);
    const int64_t tgroups = (a.N + 15) / 16;
    const int per_cu = (int)max((int64_t)1, min((int64_t)2, kLdsPerCu / (p.codes + stat)));
    int64_t grid = max((int64_t)1, min(p.groups, (int64_t)device_cus() * per_cu / tgroups));
    if (!fit_plan(a, p, grid, kLdsPerCu - stat)) return hipErrorInvalidConfiguration;
    return launch_mf(a, (int)p.nph, (int)p.qph, grid, (size_t)(p.codes + partial_bytes(p, grid)), s);
}

hipError_t launch_decode_groups(const Group *groups, int count, hipStream_t s) {
    if (count < 1 || count > kMaxMulti) return hipErrorInvalidValue;
    auto kern = decode_mfma_multi_kernel<kMfWaves, kMfSplit, kMfRing>;
    static const int64_t stat = static_lds(kern);
    if (stat < 0) return hipErrorInvalidDeviceFunction;
    GroupArgs gs[kMaxMulti];
    for (int i = 0; i < count; ++i) gs[i] = make_group_args(groups[i]);
    const int64_t N = gs[0].N;
    if (N <= 0) return hipSuccess;
    if (N > kDecodeMaxN) return hipErrorInvalidConfiguration;  // grid y
    Plan p[kMaxMulti];
    int64_t bytes[kMaxMulti], total = 0, codes_max = 0;
    for (int i = 0; i < count; ++i) {
        p[i] = plan_group(gs[i]);
        bytes[i] = group_tiles(gs[i]) * gs[i].K / 4;
        total += bytes[i];
        codes_max = max(codes_max, p[i].codes);
    }
    if (total == 0) return hipSuccess;
    const int64_t tgroups = (N + 15) / 16;
    // Workgroups per compute unit from the largest group's codes, then the
    // grid split over the groups in proportion to their weight bytes (they
    // run side by side and end together), each share raised where its
    // partial sums need it (fit_plan); one more pass if the dynamic LDS then
    // leaves room for fewer workgroups per unit.  Dynamic plus static LDS
    // stays within one compute unit's.
    int per_cu = (int)max((int64_t)1, min((int64_t)2, kLdsPerCu / (codes_max + stat)));
    int64_t grid[kMaxMulti] = {};
    int64_t shmem = 0;
    for (int pass = 0; pass < 2; ++pass) {
        // (rounded down, so that all token groups' workgroups are resident at
        // once: with 3 token groups, 86 per group put two workgroups of 258
        // into a second round -- 33 tokens of the 2B-style block 0.373 vs
        // 0.312 ms per 16 blocks, 48 of a 13B-class block 0.624 vs 0.427 ms
        // per 8)
        const int64_t budget = max((int64_t)1, (int64_t)device_cus() * per_cu / tgroups);
        shmem = 0;
        int64_t share[kMaxMulti];
        split_grid(p, bytes, count, budget, tgroups, share);
        for (int i = 0; i < count; ++i) {
            grid[i] = max((int64_t)1, min(p[i].groups, share[i]));
            if (!fit_plan(gs[i], p[i], grid[i], kLdsPerCu - stat)) return hipErrorInvalidConfiguration;
            shmem = max(shmem, p[i].codes + partial_bytes(p[i], grid[i]));
        }
        const int fit = (int)max((int64_t)1, min((int64_t)2, kLdsPerCu / (shmem + stat)));
        if (fit >= per_cu) break;
        per_cu = fit;
    }
    if (shmem + stat > kLdsPerCu) return hipErrorInvalidConfiguration;
    MultiArgs m{};
    int64_t start = 0;
    for (int i = 0; i < kMaxMulti; ++i) {
        const int j = i < count ? i : count - 1;
        m.g[i] = gs[j];
        m.nph[i] = (int)p[j].nph;
        m.qph[i] = (int)p[j].qph;
        m.start[i] = (int)start;
        if (i < count) start += grid[i];
    }
    m.start[kMaxMulti] = (int)start;
    // With several token groups every weight tile is read once per group,
    // by workgroups that sit on one XCD (the grid's width is the budget, a
    // multiple of 8): ordinary loads let the repeats hit its L2, where
    // non-temporal ones fetch them again.  Measured per block against
    // non-temporal loads: a 13B-class block at 32 / 48 tokens 1.3 / 10.4 %
    // faster, 7B-class at 32 / 64 tokens 1.3 / 1.4 %, 70B-class at 24 / 32
    // tokens 4.8 / 0.2 %, 2B-style at 96 tokens 3.0-3.7 %; but 2B-style at 33 /
    // 64 tokens 0.6-2.1 / 0.3-0.7 % slower, so blocks of at most 32 MiB keep
    // non-temporal loads below 5 token groups.  (Both instances have the same
    // static LDS: they differ only in the load instruction.)
    const bool cached = tgroups > 1 && (total > ((int64_t)32 << 20) || tgroups >= 5);
    const void *k = cached
                        ? reinterpret_cast<const void *>(
                              decode_mfma_multi_kernel<kMfWaves, kMfSplit, kMfRing, true>)
                        : reinterpret_cast<const void *>(kern);
    if (shmem > 64 * 1024) {
        const hipError_t e =
            hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess) return e;
    }
    if (cached)
        hipLaunchKernelGGL((decode_mfma_multi_kernel<kMfWaves, kMfSplit, kMfRing, true>),
                           dim3((unsigned)start, (unsigned)tgroups), dim3(kMfThreads),
                           (size_t)shmem, s, m);
    else
        hipLaunchKernelGGL(kern, dim3((unsigned)start, (unsigned)tgroups), dim3(kMfThreads),
                           (size_t)shmem, s, m);
    return hipGetLastError();
}

}  // namespace bt
