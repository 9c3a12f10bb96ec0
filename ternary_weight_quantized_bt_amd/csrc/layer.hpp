// layer.hpp -- arguments of the one-launch-per-block decode kernel (seven
// projections, four input groups).
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace bt {

constexpr int kLayerProj = BT_LAYER_PROJ;     // q, k, v, o, gate, up, down
constexpr int kLayerInputs = BT_LAYER_INPUTS;  // x0 -> q,k,v; x1 -> o; x2 -> gate,up; x3 -> down
constexpr int kLayerWaves = 16;  // waves per workgroup
constexpr int kLayerUnits = 8;   // input chunks (8 elements) held per lane in the prologue
constexpr int kLayerSpan = kWave * kLayerUnits;  // chunks per wave
// (group, token) rows one wave's span can touch: rows are at least 256
// chunks long (K >= 2048), so a 512-chunk span meets at most four.
constexpr int kWaveRows = 4;

// One wave's share of the prologue's input sequence (the four inputs seen as
// one run of 8-element chunks: input group, then token, then column), made on
// the host; the same in every workgroup.  Wave w owns chunks
// [w * kLayerSpan, (w + 1) * kLayerSpan); the chunk at span offset d lies in
// row #{r >= 1 : d >= st[r]}.  64 bytes: one scalar load per wave.
struct LayerWaveRows {
    const void *src[kWaveRows];  // element of span offset 0 in row r's layout (integer
                                 // arithmetic: may lie outside the input; only the
                                 // offsets inside row r are read through it)
    int dst[kWaveRows];          // LDS byte of span offset 0 in row r's layout
    int16_t st[kWaveRows];       // span offset where row r starts, clamped to
                                 // [-kLayerSpan, kLayerSpan] (kLayerSpan: no row)
    uint8_t key[kWaveRows];      // group * NT + token of row r (0: no row)
    int16_t nlive;               // chunks of the span inside the sequence
    int16_t nrow;                // rows that start before offset nlive (row 0 always does)
};
static_assert(sizeof(LayerWaveRows) == 64, "one 64-byte scalar load per wave");

// Workgroups whose input needs are listed (LayerArgs::need); later ones read
// all four inputs.
constexpr int kLayerNeedWgs = 256;

struct LayerArgs {
    const uint8_t *packed[kLayerProj];
    void *y[kLayerProj];
    int64_t M[kLayerProj];
    int64_t tend[kLayerProj];     // prefix sums of the projections' row tiles
    int64_t gend[kLayerInputs];   // end of each input group's tiles
    int64_t K[kLayerInputs];
    const void *x[kLayerInputs];  // float / bf16 inputs [N, K[g]]
    int64_t xoff[kLayerInputs + 1];  // LDS offset of each group's codes (rows K[g] apart)
    int64_t uoff[kLayerInputs + 1];  // first 8-element chunk of each group (all tokens)
    int64_t N;
    int ydt;
    // 32-bit copies for the kernel's scalar bookkeeping
    int tend32[kLayerProj];
    int gend32[kLayerInputs];
    int k32[kLayerInputs];
    int xoff32[kLayerInputs];
    int qb32[kLayerInputs];  // 256-column blocks per row
    // Work schedule over tile groups (the tiles one iteration of a workgroup
    // takes together).  sched = 0: workgroup w takes groups w, w + G, ...
    // sched = 1 (set by the launcher when it balances better): groups
    // [0, ts) are the light ones, [ts, end) the heavy ones; workgroups
    // [0, n0) form class 0, the rest class 1; a class-c workgroup takes an
    // even share of its class's scount[c] light groups (from sstart[c]) and
    // then heavy[c] heavy groups (class 0 from ts, class 1 from
    // ts + n0 * heavy[0]).
    int sched, n0, ts;
    int heavy[2], sstart[2], scount[2];
    // Weight format: 0 = T16Q256; 1 = base-3 B3T1024 (qb32 then counts
    // 1024-column tile columns, and the decode table sits at LDS byte tab32).
    int b3, tab32;
    const float *wscale[kLayerProj];  // each projection's weight scale (packed tail)
    const void *xlast;  // last chunk of the last input (dead lanes re-read it)
    LayerWaveRows wrows[kLayerWaves];
    // Input groups that workgroup w's tiles read: bits 4 (w % 8) .. 4 (w % 8)
    // + 3 of need[w / 8] (made with the schedule); the prologue skips the
    // spans of the others.
    uint32_t need[kLayerNeedWgs / 8];
};

// One workgroup's work under a LayerArgs schedule, shared by the kernel and
// the host-side schedule tests (so they check exactly what the kernel runs;
// the kernel passes a register view of the same fields, the host LayerArgs):
// nit iterations; in iteration it, sub-group s (of tpw) takes the row tile
// tile_for(it, s) (nothing if it is past the last tile), its waves splitting
// the tile's K blocks.
struct LayerSched {
    int nS, sfirst, nB, bfirst, nit, w, G, sched, tpw;

    template <class A>
    __host__ __device__ LayerSched(const A &a, int w_, int G_, int tpw_)
        : nS(0), sfirst(0), nB(0), bfirst(0), nit(0), w(w_), G(G_), sched(a.sched), tpw(tpw_) {
        if (sched) {
            // nS light tile groups from sfirst, then nB heavy ones from bfirst
            const int c = w < a.n0 ? 0 : 1;
            const int i = c ? w - a.n0 : w, nc = c ? G - a.n0 : a.n0;
            const int ss = c ? a.sstart[1] : a.sstart[0], sc = c ? a.scount[1] : a.scount[0];
            sfirst = ss + (int)((int64_t)i * sc / nc);
            nS = ss + (int)((int64_t)(i + 1) * sc / nc) - sfirst;
            nB = c ? a.heavy[1] : a.heavy[0];
            bfirst = a.ts + (c ? a.n0 * a.heavy[0] : 0) + i * nB;
            nit = nS + nB;
        } else {
            // every G-th tile group from w
            const int ngroups = (a.tend32[kLayerProj - 1] + tpw - 1) / tpw;
            nit = (ngroups - w + G - 1) / G;
        }
    }
    __host__ __device__ int group_of(int it) const {
        return sched ? (it < nS ? sfirst + it : bfirst + (it - nS)) : w + it * G;
    }
    __host__ __device__ int tile_for(int it, int s) const { return group_of(it) * tpw + s; }
    // K blocks of a tile of input group g (256-column blocks, or 1024-column
    // base-3 tile columns), and a wave's share kp, kp + P, ... of them.
    template <class A>
    __host__ __device__ static int blocks(const A &a, int g) {
        int q = a.qb32[0];
#pragma unroll
        for (int k = 1; k < kLayerInputs; ++k) q = g == k ? a.qb32[k] : q;
        return q;
    }
    template <class A>
    __host__ __device__ static int nq(const A &a, int g, int kp, int P) {
        return (blocks(a, g) - kp + P - 1) / P;
    }
    // Slots (blocks) that the wave with K part kpart of sub-group sub streams
    // over all its iterations, per input group in closed form.
    template <class A>
    __host__ __device__ int slots(const A &a, int sub, int kpart, int P) const {
        int n = 0;
        if (sched) {
            // tiles tg * tpw + sub for tile groups tg in [g0, g1), per input group
            auto count = [&](int g0, int g1) {
                int c = 0, prev = 0;
#pragma unroll
                for (int g = 0; g < kLayerInputs; ++g) {
                    const int end = a.gend32[g];
                    const int l0 = (prev - sub + tpw - 1) / tpw, h0 = (end - sub + tpw - 1) / tpw;
                    const int lo = g0 > l0 ? g0 : l0, hi = g1 < h0 ? g1 : h0;
                    c += hi > lo ? (hi - lo) * nq(a, g, kpart, P) : 0;
                    prev = end;
                }
                return c;
            };
            n = count(sfirst, sfirst + nS) + count(bfirst, bfirst + nB);
        } else {
            // the sequence o + it*S (it >= 0) inside each group's tile range
            const int o = w * tpw + sub, S = G * tpw;
            auto upto = [&](int x) { return x <= o ? 0 : (x - o + S - 1) / S; };
            int prev = 0;
#pragma unroll
            for (int g = 0; g < kLayerInputs; ++g) {
                const int end = a.gend32[g];
                n += (upto(end) - upto(prev)) * nq(a, g, kpart, P);
                prev = end;
            }
        }
        return n;
    }
};

// Fills the schedule fields of `a`, and the input groups each workgroup
// reads, for a grid of G workgroups (the launcher calls it; exposed for the
// host-side schedule tests).
void plan_layer_schedule(LayerArgs &a, int G, bool b3);

// Whether one launch can run the block: 1..4 tokens, every K at least one
// 256-column block per wave, all token codes in LDS and all input chunks in
// registers.
// (b3: base-3 weights, every K a multiple of 1024 and at least one tile column
// per wave of a K split, the codes within 80 KiB beside the decode table.)
bool layer_fusable(const int64_t K[kLayerInputs], const int64_t M[kLayerProj], int64_t N,
                   bt_dtype xdt, bool b3 = false);
LayerArgs make_layer_args(const uint8_t *const w[kLayerProj], const int64_t M[kLayerProj],
                          const int64_t K[kLayerInputs], const void *const x[kLayerInputs],
                          void *const y[kLayerProj], int64_t N, bt_dtype ydt, bool b3 = false);
hipError_t launch_layer(const LayerArgs &a, bt_dtype xdt, hipStream_t s);

}  // namespace bt
