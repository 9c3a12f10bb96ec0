// layer.hip -- one launch for all seven projections of a block at decode
// (a few tokens): the four inputs are quantized in the prologue and a single
// weight stream runs across every projection's row tiles.
//
// What is computed is exactly the per-group path: for each projection p with
// input group g(p) ({q,k,v} <- x0, {o} <- x1, {gate,up} <- x2, {down} <- x3),
//   y_p[n, m] = (sum_k w_p[m,k] * xq_g[n,k]) * s_w(p) * s_a(g, n) / 127
// with per-token absmax int8 codes ([PARA] section 5, Quant8 and the figure
// "BitNet b1.58 Ternary Matrix Multiplication"; [I2S] "How I2_S Kernels
// Process the Format" for the one per-tensor weight scale).  The codes and
// every output are bit-identical to the per-group launches.
//
// Why one launch.  At one token a block's projections are a few to a hundred
// MB of weights each; four dependent launches per block leave the memory
// system idle at every boundary (launch, ramp-up, the tail of the last
// tiles).  Here the workgroups walk the row tiles of all seven projections
// laid end to end (projection order q, k, v, o, gate, up, down) with a
// stride of the grid size, and each wave keeps RING slot loads in flight
// straight across tile and projection boundaries, so HBM streams from the
// first tile to the last.  The four inputs are all resident when the layer
// is called; each workgroup quantizes all of them into LDS up front.
//
// Prologue.  The inputs, seen as one sequence of 8-element chunks (input
// group, then token, then column), are dealt to the waves in contiguous
// spans of 64 x kLayerUnits chunks, lane l taking every 64th chunk from l
// (each load one contiguous KiB per wave).  A span touches only a few
// (group, token) rows (rows are >= 256 chunks long); the host lists them
// per wave in the kernel arguments, each lane keeps one running max per
// row, DPP wave reductions (quant.hpp) fold them and one lane per row folds
// the result into LDS with an atomic max.  After a barrier every chunk is
// rounded from the registers and its codes stored in LDS; code sums are
// folded the same way.  The rounding is the one of the standalone
// quantization kernel (quant.hpp), so the codes are identical.
//
// Tiles.  Within a tile the waves split K by 256-column blocks, interleaved
// (wave p of P takes blocks p, p + P, ..., so at any moment the waves of a
// tile read neighbouring KiB; every wave gets at least one block of every
// projection: K >= 256 * P).  Weight slots are loaded non-temporally (each
// byte is read once).  A lane's 16-byte slot is dotted with
// its activation words from LDS (v_dot4_i32_i8), the four lanes of a row and
// then the waves of the tile are reduced (LDS, double-buffered, one barrier
// per tile), and the epilogue dequantizes.

#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "base3.hpp"
#include "dot4.hpp"
#include "layer.hpp"
#include "quant.hpp"

namespace bt {

namespace {

constexpr int kLayerThreads = kLayerWaves * kWave;
constexpr int kLayerSplit = 8;  // K split over 8 waves: two tiles per iteration
// Slot loads in flight per wave: 3 measured fastest on the 70B-class stream
// (2 / 3 / 4 / 5 / 6: 3.34 / 3.23 / 3.31 / 3.31 / 3.33 ms per 80 blocks).
constexpr int kLayerRing = 3;
constexpr int kLayerRingB3 = 2;  // base-3 slots are 13 words
// K split of base-3 tiles (1024-column tile columns): 4 measured fastest on the
// 70B-class stream (8 / 4 / 2 / 1: 3.71 / 3.60 / 3.84 / 5.45 ms per 80 blocks;
// a third ring slot costs 3-4 %).
constexpr int kLayerSplitB3 = 4;
// Codes of all four inputs beside the 64 KiB base-3 table.
constexpr int64_t kLayerLdsMaxB3 = 80 * 1024;
// An iteration's fixed cost in base-3 tile columns (8 KiB of streaming).
constexpr int kIterCostB3 = 2;
constexpr int64_t kLayerLdsMax = 128 * 1024;  // token codes of all four inputs
constexpr int64_t kLayerMinK = (int64_t)kTileCols * kLayerSplit;  // a block per wave
static_assert(kWaveRows == kLayerSpan / (kLayerMinK / 8) + 2,
              "rows a span can touch: rows are at least kLayerMinK / 8 chunks long");

// Projection -> input group.
__host__ __device__ constexpr int proj_group(int p) { return p < 3 ? 0 : (p == 3 ? 1 : (p < 6 ? 2 : 3)); }

// arr[i] for a wave-uniform i, as a chain of selects (no dynamic indexing of
// the by-value argument block, which would move it to private memory).
template <typename T, int C>
__device__ __forceinline__ T sel(const T (&arr)[C], int i) {
    T v = arr[0];
#pragma unroll
    for (int k = 1; k < C; ++k) v = (i == k) ? arr[k] : v;
    return v;
}

// Raw input chunk of 8 elements (global loads only).
template <typename T>
struct Chunk;
template <>
struct Chunk<uint16_t> {
    v4u a;
    __device__ __forceinline__ void load(const uint16_t *p) { a = *to_global(reinterpret_cast<const v4u *>(p)); }
    __device__ __forceinline__ void clear() { a = v4u{0u, 0u, 0u, 0u}; }
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
// The kernel's view of the 32-bit bookkeeping words of LayerArgs (tend32
// through scount) held one per lane of a register (field[i] is a readlane
// with a scalar lane index), with the weight and output pointers in the
// register's upper lanes.  LayerSched reads it as it reads LayerArgs.
struct LaneWords {
    uint32_t v;
    int base;
    __device__ int operator[](int i) const { return (int)__builtin_amdgcn_readlane(v, base + i); }
};
struct BookView {
    LaneWords tend32, gend32, k32, xoff32, qb32, heavy, sstart, scount;
    int sched, n0, ts;
    __device__ explicit BookView(uint32_t v)
        : tend32{v, 0}, gend32{v, 7}, k32{v, 11}, xoff32{v, 15}, qb32{v, 19}, heavy{v, 26},
          sstart{v, 28}, scount{v, 30}, sched((int)__builtin_amdgcn_readlane(v, 23)),
          n0((int)__builtin_amdgcn_readlane(v, 24)), ts((int)__builtin_amdgcn_readlane(v, 25)) {}
    // Lanes 32..59 hold the first 28 words of LayerArgs: packed[7], then y[7].
    __device__ uint64_t word2(int i) const {
        return (uint64_t)(uint32_t)tend32[32 + i] | ((uint64_t)(uint32_t)tend32[33 + i] << 32);
    }
    __device__ const uint8_t *packed(int p) const {
        return reinterpret_cast<const uint8_t *>(word2(2 * p));
    }
    __device__ void *y(int p) const { return reinterpret_cast<void *>(word2(14 + 2 * p)); }
    // Rows of projection p, from the tile prefix sums.
    __device__ int64_t rows(int p) const {
        return (int64_t)(tend32[p] - (p > 0 ? tend32[p - 1] : 0)) * kTileRows;
    }
};
static_assert(offsetof(LayerArgs, packed) == 0 && offsetof(LayerArgs, y) == 56,
              "pointer words");
static_assert(offsetof(LayerArgs, gend32) - offsetof(LayerArgs, tend32) == 4 * 7 &&
                  offsetof(LayerArgs, k32) - offsetof(LayerArgs, tend32) == 4 * 11 &&
                  offsetof(LayerArgs, xoff32) - offsetof(LayerArgs, tend32) == 4 * 15 &&
                  offsetof(LayerArgs, qb32) - offsetof(LayerArgs, tend32) == 4 * 19 &&
                  offsetof(LayerArgs, sched) - offsetof(LayerArgs, tend32) == 4 * 23 &&
                  offsetof(LayerArgs, n0) - offsetof(LayerArgs, tend32) == 4 * 24 &&
                  offsetof(LayerArgs, ts) - offsetof(LayerArgs, tend32) == 4 * 25 &&
                  offsetof(LayerArgs, heavy) - offsetof(LayerArgs, tend32) == 4 * 26 &&
                  offsetof(LayerArgs, sstart) - offsetof(LayerArgs, tend32) == 4 * 28 &&
                  offsetof(LayerArgs, scount) - offsetof(LayerArgs, tend32) == 4 * 30,
              "bookkeeping word positions");

// B3: the weights are base-3 B3T1024 tiles (16 rows x 1024 columns, base3.hpp)
// instead of T16Q256 ones; a K split part is then a 1024-column tile column.
template <typename T, int NT, int WAVES, int P, int RING, bool B3>
__global__ __launch_bounds__(WAVES * kWave)
void layer_dot4_kernel(LayerArgs a) {
    static_assert(WAVES % P == 0, "K split must divide the waves");
    static_assert(16 * NT <= kWave, "one wave stores a tile");
    static_assert(kLayerProj <= WAVES, "one wave per weight scale");
    constexpr int TPW = WAVES / P;
    constexpr int kKeys = kLayerInputs * NT;
    extern __shared__ __attribute__((aligned(16))) int8_t codes[];
    __shared__ int red[2][WAVES][NT][16];
    __shared__ uint32_t s_amax[kKeys];  // max |x| bits per (group, token)
    __shared__ uint32_t s_sum[kKeys];   // code sum per (group, token)
    __shared__ float s_ws[kLayerProj];  // weight scales

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // The argument block is read throughout the setup below in chains of
    // dependent scalar loads, and it starts every launch outside the scalar
    // cache: touch each 64-byte line of its head and this wave's row table
    // first, all loads in flight together, so the chains then hit the cache
    // instead of paying a miss per line in turn.
    // The wave's row table is read in the same batch, as 16 words (its
    // 16-bit fields sit at offsets a scalar load cannot take on their own).
    // So is the word listing the inputs this workgroup reads.
    uint32_t wt[16];
    uint32_t needw;
    {
        const auto *ka = (const __attribute__((address_space(4))) uint32_t *)
            __builtin_amdgcn_kernarg_segment_ptr();
        constexpr int kWords = (int)(offsetof(LayerArgs, wrows) / 4);
        static_assert(kWords <= 160, "ten 64-byte lines");
        static_assert(offsetof(LayerArgs, wrows) % 4 == 0, "word-aligned row tables");
        uint32_t t[10];
#pragma unroll
        for (int i = 0; i < 10; ++i) t[i] = ka[min(16 * i, kWords - 1)];
        const auto *kw = ka + kWords + 16 * wave;
#pragma unroll
        for (int i = 0; i < 16; ++i) wt[i] = kw[i];
        needw = ka[offsetof(LayerArgs, need) / 4 + min((int)blockIdx.x, kLayerNeedWgs - 1) / 8];
        asm volatile("" : : "s"(t[0]), "s"(t[1]), "s"(t[2]), "s"(t[3]), "s"(t[4]),
                     "s"(t[5]), "s"(t[6]), "s"(t[7]), "s"(t[8]), "s"(t[9]), "s"(needw));
        asm volatile("" : : "s"(wt[0]), "s"(wt[1]), "s"(wt[2]), "s"(wt[3]), "s"(wt[4]),
                     "s"(wt[5]), "s"(wt[6]), "s"(wt[7]), "s"(wt[8]), "s"(wt[9]),
                     "s"(wt[10]), "s"(wt[11]), "s"(wt[12]), "s"(wt[13]), "s"(wt[14]),
                     "s"(wt[15]));
    }
    // The schedule's 32-bit words (tend32 .. scount) in lanes 0..31 and the
    // weight and output pointers (packed[], y[]) in lanes 32..59 of one
    // register, by ONE vector load issued ahead of the input loads; every
    // lookup is then a readlane with a scalar index.  Read through the scalar
    // cache, the setup's lookups were chains of dependent loads, each waited
    // for, in all 16 waves of the unit: the first barrier came 2.1 us after
    // the input loads went out, and a 2560/6912 block at one token took
    // 11.95 us against 11.56 us now (70B-class: 0.2 % in alternating runs).
    static_assert(offsetof(LayerArgs, scount) + 8 - offsetof(LayerArgs, tend32) == 4 * 32,
                  "32 bookkeeping words");
    uint32_t bkv;
    {
        const auto *k0 = reinterpret_cast<const uint32_t *>(
            reinterpret_cast<uintptr_t>(__builtin_amdgcn_kernarg_segment_ptr()));
        const auto *kb = k0 + offsetof(LayerArgs, tend32) / 4;
        bkv = *to_global(lane < 32 ? kb + lane : k0 + min(lane - 32, 27));
    }
    const BookView bk(bkv);
    const int h = lane / 16;
    const int nvalid = (int)min((int64_t)NT, a.N);
    const int kpart = wave % P, sub = wave / P;
    // ---- prologue, part 1: this wave's input chunks into registers ----
    // Lane l holds chunks w * kLayerSpan + 64c + l (c < kLayerUnits) of the
    // sequence, so every load is one contiguous KiB per wave; the rows the
    // span touches come from the wave's table (LayerWaveRows, made on the
    // host).
    static_assert(offsetof(LayerWaveRows, src) == 0 && offsetof(LayerWaveRows, dst) == 32 &&
                      offsetof(LayerWaveRows, st) == 48 && offsetof(LayerWaveRows, key) == 56 &&
                      offsetof(LayerWaveRows, nlive) == 60 && offsetof(LayerWaveRows, nrow) == 62,
                  "row table words");
    const int nrow = (int16_t)(wt[15] >> 16);
    const T *rsrc[kWaveRows];  // element of span offset 0 in row r's layout
    int rdst[kWaveRows];       // LDS byte of span offset 0 in row r's layout
    int rkey[kWaveRows];       // group * NT + token of row r
    int st[kWaveRows];         // span offset where row r starts
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) {
        rsrc[r] = reinterpret_cast<const T *>(((uint64_t)wt[2 * r + 1] << 32) | wt[2 * r]);
        rdst[r] = (int)wt[8 + r];
        rkey[r] = (int)((wt[14] >> (8 * r)) & 0xFFu);
        st[r] = (int16_t)((wt[12 + r / 2] >> (16 * (r % 2))) & 0xFFFFu);
    }
    // A span lying only in inputs that none of this workgroup's tiles read
    // is skipped: no loads, no codes (its LDS is never read).
    const uint32_t need = blockIdx.x < kLayerNeedWgs ? (needw >> (4 * (blockIdx.x % 8))) & 0xFu : 0xFu;
    bool wanted = false;
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) wanted |= r < nrow && ((need >> (rkey[r] / NT)) & 1u) != 0;
    const int nlive = wanted ? (int16_t)(wt[15] & 0xFFFFu) : 0;
    // Dead lanes (past the sequence) re-read the last chunk of the last row;
    // a wave with no live chunk issues no load (the prologue's loads queue
    // behind one another, and at one 70B-class token three of the 16 waves
    // hold nothing).
    const T *last = static_cast<const T *>(a.xlast);
    Chunk<T> raw[kLayerUnits];
    int rowof[kLayerUnits];
    if (nlive == 0) {
#pragma unroll
        for (int c = 0; c < kLayerUnits; ++c) {
            raw[c].clear();
            rowof[c] = 0;
        }
    } else {
#pragma unroll
        for (int c = 0; c < kLayerUnits; ++c) {
            const int d = kWave * c + lane;
            int r = 0;
            const T *src = rsrc[0];
#pragma unroll
            for (int k = 1; k < kWaveRows; ++k) {
                r += d >= st[k] ? 1 : 0;
                src = d >= st[k] ? rsrc[k] : src;
            }
            raw[c].load(d < nlive ? src + 8 * d : last);
            rowof[c] = r;
        }
    }
    if (threadIdx.x < kKeys) {
        s_amax[threadIdx.x] = 0;
        s_sum[threadIdx.x] = 0;
    }

    // Tile bookkeeping in 32-bit scalars: tile and slot counts are far below
    // 2^31, and 64-bit compares would run on the vector unit.
    const int total = bk.tend32[kLayerProj - 1];
    // This workgroup's tile groups (see LayerArgs::sched and LayerSched): nS
    // light ones from sfirst, then nB heavy ones from bfirst; or every G-th
    // from w.
    const int G = (int)gridDim.x, w = (int)blockIdx.x;
    const LayerSched ls(bk, w, G, TPW);
    const int nit = ls.nit;
    auto group_of = [&](int it) { return ls.group_of(it); };
    auto tile_of = [&](int it) { return group_of(it) * TPW + sub; };
    // This wave's blocks in a tile of input group g: kpart, kpart + P, ...
    // (interleaved, so the waves of a tile read neighbouring KiB together),
    // nq(g) of them, at least one (K >= 256 * P).
    auto nq = [&](int g) { return (bk.qb32[g] - kpart + P - 1) / P; };
    // Projection of a tile index that only grows (each cursor below walks
    // its tiles in order): re-resolved only when the tile leaves the current
    // projection's tile range [start, end).
    struct Win {
        int p, start, end;
    };
    auto win0 = [&]() { return Win{0, 0, bk.tend32[0]}; };
    auto seek = [&](Win &w, int t) {
        while (t >= w.end) {
            ++w.p;
            w.start = w.end;
            w.end = bk.tend32[w.p];
        }
    };

    // Slots of this wave: nq(g) per tile of input group g among its tiles.
    const int nslots = ls.slots(bk, sub, kpart, P);
    const bool has_work = nit > 0 && tile_of(0) < total;

    // Load cursor: tile iteration lit, lrem slots left in its tile (the
    // current one included), lleft slots left to load.  On the last slot it
    // stays put, so every ring load is unconditional (a harmless reload).
    int lit = 0, lrem = 0, lleft = nslots;
    const uint8_t *lp = nullptr;  // T16Q256: the slot (wave-uniform)
    const uint8_t *lt = nullptr;  // B3T1024: the tile
    Win lw = win0();
    int lnq = 0, lqb = 0;
    const uint8_t *lbase = nullptr;
    auto point = [&](int t) {
        if (t >= lw.end || lbase == nullptr) {
            seek(lw, t);
            const int g = proj_group(lw.p);
            lnq = nq(g);
            lqb = bk.qb32[g];
            lbase = bk.packed(lw.p);
        }
        lrem = lnq;
        if constexpr (B3)
            lt = lbase + ((int64_t)(t - lw.start) * lqb + kpart) * kB3TileBytes;
        else
            lp = lbase + ((int64_t)(t - lw.start) * lqb + kpart) * kTileBytes;
    };
    point(has_work ? tile_of(0) : 0);
    auto advance_load = [&]() {
        if (lleft <= 1) return;
        --lleft;
        if (--lrem > 0) {
            if constexpr (B3)
                lt += (int64_t)kB3TileBytes * P;
            else
                lp += (int64_t)kTileBytes * P;
            return;
        }
        point(tile_of(++lit));
    };
    using Slot = typename std::conditional<B3, B3Slot, v4u>::type;
    auto load = [&]() -> Slot {
        if constexpr (B3)
            return load_slot<true>(lt, lane);
        else
            return __builtin_nontemporal_load(to_global(reinterpret_cast<const v4u *>(lp)) + lane);
    };
    constexpr int kSlots = RING + 1;
    Slot ring[kSlots];
    // Base-3 tiles: the ring's first slots go out now, before the table is
    // built (later costs 0.4 % on the 70B-class stream); 2-bit tiles issue
    // them after the absmax barrier, below.
    if constexpr (B3) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            ring[d] = load();
            advance_load();
        }
    }
    if constexpr (B3)
        b3_build_table(reinterpret_cast<uint8_t *>(codes) + a.tab32, (int)threadIdx.x,
                       (int)(WAVES * kWave));
    __syncthreads();  // zeroed tables

    // ---- prologue, part 2: absmax per (group, token) ----
    if (nrow == 1) {
        // the whole span lies in one row (the common case for long rows)
        uint32_t m = 0;
#pragma unroll
        for (int c = 0; c < kLayerUnits; ++c)
            m = max(m, kWave * c + lane < nlive ? raw[c].abs_bits() : 0u);
        const uint32_t mw = wave_reduce<true>(m);
        if (lane == 0) atomicMax(&s_amax[rkey[0]], mw);
    } else {
        uint32_t mx[kWaveRows] = {};
#pragma unroll
        for (int c = 0; c < kLayerUnits; ++c) {
            const uint32_t v = kWave * c + lane < nlive ? raw[c].abs_bits() : 0u;
#pragma unroll
            for (int r = 0; r < kWaveRows; ++r) mx[r] = rowof[c] == r ? max(mx[r], v) : mx[r];
        }
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r) {
            if (r < nrow) {
                const uint32_t m = wave_reduce<true>(mx[r]);
                if (lane == 0) atomicMax(&s_amax[rkey[r]], m);
            }
        }
    }
    // every input chunk has landed (absmax read them all): say so, so that
    // the quantization below needs no wait that would also cover the scale
    // and ring loads issued next
    if constexpr (!B3) __builtin_amdgcn_s_waitcnt(0x3F70);
    __syncthreads();
    // Weight scales, one per projection in its packed tail (addresses made
    // on the host): lane p < 7 of wave 0 loads scale p, after the input
    // loads, and it is waited for only where the scales go to LDS at the end
    // of the prologue.  The seven addresses are opaque scalars picked per
    // lane, so no indexed load of the argument block sits in front of it.
    float wsl = 0.0f;
    if (wave == 0) {
        const float *sp = a.wscale[0];
#pragma unroll
        for (int k = 1; k < kLayerProj; ++k) {
            const float *q = a.wscale[k];
            asm volatile("" : "+s"(q));
            sp = lane == k ? q : sp;
        }
        wsl = *to_global(sp);
    }

    // The first 2-bit weight slots go out here, behind the input loads: issued
    // before the first barrier they queue with the input loads and hold up
    // every wave's arrival there (the vector-memory queue is full at that
    // point); here they still arrive before the quantization is done.
    // (Measured on the 70B-class stream against issuing them before the
    // first barrier / after it / after the prologue: 3.180 vs 3.196 / 3.187 /
    // 3.261 ms per 80 blocks.)
    if constexpr (!B3) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            ring[d] = load();
            advance_load();
        }
    }

    // ---- prologue, part 3: codes into LDS, code sums ----
    const float inv0 = quant_inv(__uint_as_float(s_amax[rkey[0]]));
    if (nrow == 1 && !__builtin_isinf(inv0)) {
        int sum = 0;
#pragma unroll
        for (int c = 0; c < kLayerUnits; ++c) {
            const int d = kWave * c + lane;
            int part = 0;
            const uint2 q = quant8_finite(raw[c].eight(), inv0, part);
            if (d < nlive) {
                *reinterpret_cast<uint2 *>(codes + rdst[0] + 8 * d) = q;
                sum += part;
            }
        }
        const uint32_t sw = wave_reduce<false>((uint32_t)sum);
        if (lane == 0) atomicAdd(&s_sum[rkey[0]], sw);
    } else {
        // the span crosses rows (short rows), or 127 / amax overflows
        float inv[kWaveRows];
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r) inv[r] = quant_inv(__uint_as_float(s_amax[rkey[r]]));
        int sm[kWaveRows] = {};
#pragma unroll
        for (int c = 0; c < kLayerUnits; ++c) {
            const int d = kWave * c + lane;
            const int r = rowof[c];
            float iv = inv[0];
            int base = rdst[0];
#pragma unroll
            for (int k = 1; k < kWaveRows; ++k) {
                iv = r == k ? inv[k] : iv;
                base = r == k ? rdst[k] : base;
            }
            int part = 0;
            const uint2 q = quant8(raw[c].eight(), iv, part);
            if (d < nlive) {
                *reinterpret_cast<uint2 *>(codes + base + 8 * d) = q;
#pragma unroll
                for (int k = 0; k < kWaveRows; ++k) sm[k] += r == k ? part : 0;
            }
        }
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r) {
            if (r < nrow) {
                const uint32_t sum = wave_reduce<false>((uint32_t)sm[r]);
                if (lane == 0) atomicAdd(&s_sum[rkey[r]], sum);
            }
        }
    }
    if (wave == 0 && lane < kLayerProj) s_ws[lane] = wsl;
    __syncthreads();

    // ---- tiles ----
    // Compute cursor: iteration cit, block cq (stepping by P) of its tile,
    // crem slots left in it, whose input group's codes start at xb.
    int cit = 0, cq = 0, crem = 0, cK = 0, cnq = 0;
    const int8_t *xb = codes;
    Win cw = win0();
    bool cfirst = true;
    auto enter = [&](int it) {
        const int t = tile_of(it);
        if (t >= total) return;
        if (t >= cw.end || cfirst) {
            seek(cw, t);
            const int g = proj_group(cw.p);
            cnq = nq(g);
            cK = bk.k32[g];
            xb = codes + bk.xoff32[g] + (B3 ? 256 : 16) * h;
            cfirst = false;
        }
        cq = kpart;
        crem = cnq;
    };
    enter(0);

    int buf = 0;
    Win ow = win0();  // the tiles this wave stores (waves < TPW)
    Acc<NT> acc;
    acc_zero(acc);
    int iacc[NT];  // B3 sums
#pragma unroll
    for (int j = 0; j < NT; ++j) iacc[j] = 0;
    const uint8_t *tab = reinterpret_cast<const uint8_t *>(codes) + a.tab32;
    const uint32_t l8 = 8u * (uint32_t)(lane % kB3Copies);
    auto iter_done = [&](int it) {
        int v[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if constexpr (B3) {
                v[j] = iacc[j];
                iacc[j] = 0;
            } else {
                v[j] = acc_total(acc, j);
            }
            v[j] += __shfl_xor(v[j], 16, kWave);
            v[j] += __shfl_xor(v[j], 32, kWave);
        }
        acc_zero(acc);
        if (lane < 16) {
#pragma unroll
            for (int j = 0; j < NT; ++j) red[buf][wave][j][lane] = v[j];
        }
        __syncthreads();
        // wave s (< TPW) stores the tile of sub-group s: lane = 16 * token + row
        // (the tile is wave-uniform, so its projection is resolved in scalars)
        if (wave < TPW) {
            const int s = wave;
            const int j = lane / 16, r = lane % 16;
            const int tile = group_of(it) * TPW + s;
            if (tile < total) {
                seek(ow, tile);
                if (j < nvalid) {
                    const int p = ow.p, g = proj_group(p);
                    int t = 0;
#pragma unroll
                    for (int q = 0; q < P; ++q) t += red[buf][s * P + q][j][r];
                    const int64_t M = bk.rows(p);
                    const float f = token_factor(s_ws[p], __uint_as_float(s_amax[g * NT + j]));
                    store_out(bk.y(p), a.ydt, j * M + (int64_t)(tile - ow.start) * kTileRows + r,
                              t - (int32_t)s_sum[g * NT + j], f);
                }
            }
        }
        buf ^= 1;
    };

    if (!has_work) {
        for (int it = 0; it < nit; ++it) iter_done(it);
        return;
    }
    for (int base = 0; base < nslots; base += kSlots) {
#pragma unroll
        for (int d = 0; d < kSlots; ++d) {
            const int i = base + d;
            if (i < nslots) {
                if constexpr (B3)
                    b3_dot<NT>(ring[d], tab, l8, xb + cq * kB3Cols, cK, nvalid, iacc);
                else
                    dot_slot<NT>(ring[d], xb + cq * kTileCols, cK, nvalid, acc);
            }
            ring[(d + RING) % kSlots] = load();
            advance_load();
            if (i < nslots) {
                cq += P;
                if (--crem == 0) {
                    iter_done(cit);
                    enter(++cit);
                }
            }
        }
    }
    // Iterations whose tile for this wave's sub-group is past the end (the
    // other sub-groups' last tiles) still need this wave at the barrier.
    for (; cit < nit; ++cit) iter_done(cit);
}

// A balanced schedule for the common shape of a block: tile groups of two
// weights (the light ones, e.g. every projection with K = hidden) followed
// by heavier ones (the down projection, K = FFN width).  Striding over the
// groups gives every workgroup the same number of them, give or take one,
// so with G workgroups the last round decides the time; two classes of
// workgroups -- y0 heavy groups plus up to x0 light ones, or y1 heavy plus
// up to x1 light -- can do better.  The smallest bound B (in 256-column
// blocks) for which such a split exists is found by a short scan; the
// schedule is used only if it beats striding.  Costs are blocks streamed.
// Fixed cost of one iteration (reduction, barrier, stores) in blocks of
// streaming, for the schedule's cost model.  Measured on the 70B-class
// block: 0, 8, 32 and 64 give 1.3 %, 1.9 %, -5 % and -0.8 % against striding.
constexpr int kIterCostBlocks = 8;

// iter_cost: the same fixed cost in the schedule's units (256-column blocks,
// or 1024-column base-3 tile columns: 3.25 KiB each).
template <int TPW>
void plan_schedule(LayerArgs &a, int G, int iter_cost) {
    a.sched = 0;
    const int total = a.tend32[kLayerProj - 1];
    const int T = (total + TPW - 1) / TPW;
    if (G <= 0 || T <= G) return;  // at most one group per workgroup
    auto tile_cost = [&](int t) {
        if (t >= total) return 0;
        int g = 0;
        while (t >= a.gend32[g]) ++g;
        return a.qb32[g];
    };
    auto group_cost = [&](int tg) {
        int c = iter_cost;
        for (int k = 0; k < TPW; ++k) c += tile_cost(tg * TPW + k);
        return c;
    };
    const int64_t ca = group_cost(0);
    int ts = 1;
    while (ts < T && group_cost(ts) == ca) ++ts;
    if (ts == T) return;  // one kind of group
    const int64_t cb = group_cost(ts);
    if (cb <= ca) return;
    for (int tg = ts + 1; tg < T; ++tg)
        if (group_cost(tg) != cb) return;  // more than two kinds: keep striding
    const int64_t nA = ts, nB = T - ts;
    // cost of the slowest workgroup when striding
    int64_t stride_max = 0;
    for (int w = 0; w < G; ++w) {
        const int64_t na = w < nA ? (nA - w + G - 1) / G : 0;
        const int64_t first_b = (ts - w + G - 1) / G * G + w;  // first tg >= ts with tg % G == w
        const int64_t nb = first_b < T ? (T - first_b + G - 1) / G : 0;
        stride_max = std::max(stride_max, na * ca + nb * cb);
    }
    const int64_t lb = (nA * ca + nB * cb + G - 1) / G;
    for (int64_t B = lb; B < stride_max; ++B) {
        for (int64_t y0 = 0; y0 * cb <= B; ++y0) {
            for (int64_t y1 = y0; y1 * cb <= B; ++y1) {
                const int64_t x0 = (B - y0 * cb) / ca, x1 = (B - y1 * cb) / ca;
                int64_t n0, n1;
                if (y1 == y0) {
                    if (y0 * G != nB) continue;
                    n0 = G;
                    n1 = 0;
                } else {
                    if ((nB - y0 * G) % (y1 - y0) != 0) continue;
                    n1 = (nB - y0 * G) / (y1 - y0);
                    n0 = G - n1;
                    if (n1 < 0 || n0 < 0) continue;
                }
                if (x0 * n0 + x1 * n1 < nA) continue;
                // light groups per class: as even per-workgroup costs as the
                // caps allow
                int64_t s0 = nA;
                if (n1 > 0 && n0 > 0) {
                    const double t = ((double)nA / n1 + (double)cb / ca * (y1 - y0)) / (1.0 / n0 + 1.0 / n1);
                    s0 = std::min(std::max((int64_t)(t + 0.5), nA - x1 * n1), std::min(nA, x0 * n0));
                } else if (n0 == 0) {
                    s0 = 0;
                }
                const int64_t s1 = nA - s0;
                const int64_t m0 = n0 ? (s0 + n0 - 1) / n0 * ca + y0 * cb : 0;
                const int64_t m1 = n1 ? (s1 + n1 - 1) / n1 * ca + y1 * cb : 0;
                if (std::max(m0, m1) >= stride_max) continue;
                a.sched = 1;
                a.n0 = (int)n0;
                a.ts = ts;
                a.heavy[0] = (int)y0;
                a.heavy[1] = (int)y1;
                a.sstart[0] = 0;
                a.scount[0] = (int)s0;
                a.sstart[1] = (int)s0;
                a.scount[1] = (int)s1;
                return;
            }
        }
    }
}

template <typename T, int NT, bool B3>
hipError_t launch_layer_t(const LayerArgs &args, size_t lds, hipStream_t s) {
    constexpr int P = B3 ? kLayerSplitB3 : kLayerSplit;
    auto kern = layer_dot4_kernel<T, NT, kLayerWaves, P, B3 ? kLayerRingB3 : kLayerRing, B3>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    constexpr int TPW = kLayerWaves / P;
    const int64_t groups = (args.tend[kLayerProj - 1] + TPW - 1) / TPW;
    const int64_t grid = min(groups, (int64_t)device_cus());
    LayerArgs a = args;
    plan_layer_schedule(a, (int)grid, B3);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kLayerThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

void plan_layer_schedule(LayerArgs &a, int G, bool b3) {
    if (b3)
        plan_schedule<kLayerWaves / kLayerSplitB3>(a, G, kIterCostB3);
    else
        plan_schedule<kLayerWaves / kLayerSplit>(a, G, kIterCostBlocks);
    // The input groups each workgroup's tiles read.  Under the two-class
    // schedule a workgroup's tiles are two contiguous ranges, each spanning
    // the groups from its first tile's to its last tile's; a striding
    // workgroup with few iterations is walked, one with many reads all four.
    const int tpw = kLayerWaves / (b3 ? kLayerSplitB3 : kLayerSplit);
    const int total = a.tend32[kLayerProj - 1];
    auto group_of_tile = [&](int t) {
        int g = 0;
        while (g + 1 < kLayerInputs && t >= a.gend32[g]) ++g;
        return g;
    };
    auto range = [&](int g0, int n) -> uint32_t {  // tile groups [g0, g0 + n)
        const int t0 = g0 * tpw, t1 = std::min((g0 + n) * tpw, total);
        if (n <= 0 || t0 >= t1) return 0u;
        const int lo = group_of_tile(t0), hi = group_of_tile(t1 - 1);
        return ((2u << hi) - 1u) & ~((1u << lo) - 1u);
    };
    for (auto &x : a.need) x = 0u;
    for (int w = 0; w < std::min(G, kLayerNeedWgs); ++w) {
        const LayerSched ls(a, w, G, tpw);
        uint32_t m = 0u;
        if (ls.sched) {
            m = range(ls.sfirst, ls.nS) | range(ls.bfirst, ls.nB);
        } else if ((int64_t)ls.nit * tpw <= 64) {
            for (int it = 0; it < ls.nit; ++it)
                for (int sg = 0; sg < tpw; ++sg) {
                    const int t = ls.tile_for(it, sg);
                    if (t < total) m |= 1u << group_of_tile(t);
                }
        } else {
            m = 0xFu;
        }
        a.need[w / 8] |= m << (4 * (w % 8));
    }
}

// Largest 2-bit block (packed bytes) that the one-launch kernel takes at N
// tokens.  From 2 tokens on its dot4 products read every token's activation
// words from LDS for each weight slot (four 16-byte reads per token), so its
// time grows with N times the weight bytes, while the four-group matrix-core
// decode (plus one quantization launch) costs a fixed ~14 us plus the
// stream.  Measured per block (us, one-launch vs matrix cores): 2 tokens:
// 11.3 MB 12.0 vs 15.3, 50.6 MB 19.8 vs 21.3, 79.3 MB 25.3 vs 24.4; 3 tokens:
// 11.3 MB 13.2 vs 15.6, 17.4 MB 16.2 vs 16.9; 4 tokens: 11.3 MB 15.2 vs 15.7,
// 17.4 MB 18.9 vs 16.7.
static int64_t fused_max_bytes(int64_t N) {
    constexpr int64_t kMB = 1000000;
    return N <= 1 ? INT64_MAX : N == 2 ? 64 * kMB : N == 3 ? 20 * kMB : 12 * kMB;
}

bool layer_fusable(const int64_t K[kLayerInputs], const int64_t M[kLayerProj], int64_t N,
                   bt_dtype xdt, bool b3) {
    if (N < 1 || N > 4) return false;
    if (xdt != BT_BF16) return false;  // f32 chunks would need twice the registers
    int64_t sumk = 0;
    for (int g = 0; g < kLayerInputs; ++g) {
        if (K[g] < kLayerMinK) return false;
        if (b3 && (K[g] % kB3Cols != 0 || K[g] < (int64_t)kB3Cols * kLayerSplitB3)) return false;
        sumk += K[g];
    }
    int64_t tiles = 0, bytes = 0;
    for (int p = 0; p < kLayerProj; ++p) {
        tiles += M[p] / kTileRows;
        bytes += M[p] * K[proj_group(p)] / 4;
    }
    if (tiles >= (int64_t)1 << 30) return false;  // tile bookkeeping is 32-bit
    // (base-3 blocks have no matrix-core path: the one launch is their fastest)
    if (!b3 && bytes > fused_max_bytes(N)) return false;
    const int nt = N == 1 ? 1 : (N == 2 ? 2 : 4);
    if (nt * sumk > (b3 ? kLayerLdsMaxB3 : kLayerLdsMax)) return false;
    const int64_t units = N * sumk / 8;
    return units <= (int64_t)kLayerUnits * kLayerThreads;
}

LayerArgs make_layer_args(const uint8_t *const w[kLayerProj], const int64_t M[kLayerProj],
                          const int64_t K[kLayerInputs], const void *const x[kLayerInputs],
                          void *const y[kLayerProj], int64_t N, bt_dtype ydt, bool b3) {
    LayerArgs a{};
    int64_t end = 0;
    for (int p = 0; p < kLayerProj; ++p) {
        a.packed[p] = w[p];
        a.y[p] = y[p];
        a.M[p] = M[p];
        end += M[p] / kTileRows;
        a.tend[p] = end;
    }
    a.gend[0] = a.tend[2];
    a.gend[1] = a.tend[3];
    a.gend[2] = a.tend[5];
    a.gend[3] = a.tend[6];
    const int nt = N == 1 ? 1 : (N == 2 ? 2 : 4);
    int64_t xo = 0, uo = 0;
    for (int g = 0; g < kLayerInputs; ++g) {
        a.K[g] = K[g];
        a.x[g] = x[g];
        a.xoff[g] = xo;
        a.uoff[g] = uo;
        xo += nt * K[g];
        uo += N * K[g] / 8;
    }
    a.xoff[kLayerInputs] = xo;
    a.uoff[kLayerInputs] = uo;
    for (int p = 0; p < kLayerProj; ++p) a.tend32[p] = (int)a.tend[p];
    for (int g = 0; g < kLayerInputs; ++g) {
        a.gend32[g] = (int)a.gend[g];
        a.k32[g] = (int)a.K[g];
        a.xoff32[g] = (int)a.xoff[g];
        a.qb32[g] = (int)(a.K[g] / (b3 ? kB3Cols : kTileCols));
    }
    a.N = N;
    a.ydt = (int)ydt;
    a.b3 = b3 ? 1 : 0;
    a.tab32 = (int)((xo + 15) / 16 * 16);  // base-3 table after the codes
    for (int p = 0; p < kLayerProj; ++p) {
        const int64_t Kp = a.K[proj_group(p)];
        a.wscale[p] = reinterpret_cast<const float *>(
            w[p] + (b3 ? b3_code_bytes(M[p], Kp) : M[p] * Kp / 4));
    }
    // The inputs are bf16 (layer_fusable); the prologue's tables address them
    // in 2-byte elements.
    constexpr int64_t kElem = 2;
    a.xlast = reinterpret_cast<const void *>(reinterpret_cast<uintptr_t>(x[kLayerInputs - 1]) +
                                             (uintptr_t)((N * K[kLayerInputs - 1] - 8) * kElem));
    // Each wave's span of the chunk sequence: the row holding its first chunk
    // (the last chunk of the sequence for a span past the end), then the rows
    // that follow it, kWaveRows in all (past the fourth input: no row).
    const int64_t units = uo;
    for (int wv = 0; wv < kLayerWaves; ++wv) {
        LayerWaveRows &t = a.wrows[wv];
        const int64_t u0 = (int64_t)wv * kLayerSpan;
        const int64_t nlive = std::max<int64_t>(0, std::min<int64_t>(kLayerSpan, units - u0));
        const int64_t u = std::min(u0, units - 1);
        int g = 0;
        while (g + 1 < kLayerInputs && u >= a.uoff[g + 1]) ++g;
        int64_t cpr = K[g] / 8;
        int64_t j = (u - a.uoff[g]) / cpr;
        int64_t start = a.uoff[g] + j * cpr - u0;  // <= 0
        int nrow = 0;
        for (int r = 0; r < kWaveRows; ++r) {
            const bool real = g < kLayerInputs;
            const int gg = real ? g : kLayerInputs - 1;
            // span offsets d only meet st[r] for r >= 1, where 0 < start; any
            // value >= kLayerSpan compares like "no row"
            t.st[r] = (int16_t)(real ? std::min<int64_t>(std::max<int64_t>(start, -kLayerSpan), kLayerSpan)
                                     : kLayerSpan);
            t.key[r] = (uint8_t)(real ? g * nt + j : 0);
            t.src[r] = reinterpret_cast<const void *>(reinterpret_cast<uintptr_t>(x[gg]) +
                                                      (uintptr_t)((j * K[gg] - 8 * start) * kElem));
            t.dst[r] = (int)(a.xoff[gg] + j * K[gg] - 8 * start);
            nrow += (real && start < nlive) ? 1 : 0;
            start += cpr;
            if (++j == N) {
                j = 0;
                ++g;
                cpr = g < kLayerInputs ? K[g] / 8 : 1;
            }
        }
        t.nlive = (int16_t)nlive;
        t.nrow = (int16_t)nrow;
    }
    return a;
}

hipError_t launch_layer(const LayerArgs &a, bt_dtype xdt, hipStream_t s) {
    if (xdt != BT_BF16) return hipErrorInvalidValue;  // excluded by layer_fusable
    if (a.b3) {
        const size_t lds = (size_t)a.tab32 + kB3TabBytes;
        if (a.N == 1) return launch_layer_t<uint16_t, 1, true>(a, lds, s);
        if (a.N == 2) return launch_layer_t<uint16_t, 2, true>(a, lds, s);
        return launch_layer_t<uint16_t, 4, true>(a, lds, s);
    }
    const size_t lds = (size_t)a.xoff[kLayerInputs];
    if (a.N == 1) return launch_layer_t<uint16_t, 1, false>(a, lds, s);
    if (a.N == 2) return launch_layer_t<uint16_t, 2, false>(a, lds, s);
    return launch_layer_t<uint16_t, 4, false>(a, lds, s);
}

}  // namespace bt
