// layer.hpp -- arguments of the one-launch-per-block decode kernel (seven
// projections, four input groups).
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace bt {

constexpr int kLayerProj = BT_LAYER_PROJ;     // q, k, v, o, gate, up, down
constexpr int kLayerInputs = BT_LAYER_INPUTS;  // x0 -> q,k,v; x1 -> o; x2 -> gate,up; x3 -> down

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
};

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
