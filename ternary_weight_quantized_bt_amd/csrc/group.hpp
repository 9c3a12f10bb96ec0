// group.hpp -- kernel-side view of a grouped launch: up to three projections
// that share the same quantized input (q/k/v or gate/up) run in one grid,
// their 16-row tiles laid end to end.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace bt {

struct GroupArgs {
    const uint8_t *packed[kMaxGroup];
    void *y[kMaxGroup];
    int64_t M[kMaxGroup];
    int64_t tiles_end[kMaxGroup];  // prefix sums of M/16; unused = total
    int64_t K;
    const int8_t *xq;
    const float *xs;
    const int32_t *xsum;
    int64_t N;
    int ydt;
};

inline GroupArgs make_group_args(const Group &g) {
    GroupArgs a{};
    int64_t end = 0;
    for (int i = 0; i < kMaxGroup; ++i) {
        if (i < g.count) {
            a.packed[i] = g.p[i].packed;
            a.y[i] = g.p[i].y;
            a.M[i] = g.p[i].M;
            end += g.p[i].M / kTileRows;
        } else {
            a.packed[i] = g.p[0].packed;
            a.y[i] = g.p[0].y;
            a.M[i] = g.p[0].M;
        }
        a.tiles_end[i] = end;
    }
    a.K = g.K;
    a.xq = g.xq;
    a.xs = g.xs;
    a.xsum = g.xsum;
    a.N = g.N;
    a.ydt = (int)g.ydt;
    return a;
}

__host__ __device__ inline int64_t group_tiles(const GroupArgs &a) { return a.tiles_end[kMaxGroup - 1]; }

// The projection a global row tile belongs to, and its local row tile.
struct TileRef {
    const uint8_t *packed;
    void *y;
    int64_t M;
    int64_t mt;
    int proj;  // index of the projection within the group
};

// Branch-free pick among three loaded values with all-ones / all-zeros masks.
// Selecting between the values (rather than between their addresses) keeps
// the by-value argument struct out of private memory.
__device__ __forceinline__ uint64_t pick3(uint64_t m1, uint64_t m2, uint64_t v0,
                                          uint64_t v1, uint64_t v2) {
    return (v0 & ~m1) | (v1 & m1 & ~m2) | (v2 & m2);
}

// Weight scale of projection p of the group (read from its packed tail).
__device__ __forceinline__ float group_weight_scale(const GroupArgs &a, int p) {
    const uint64_t m1 = p >= 1 ? ~0ull : 0ull, m2 = p >= 2 ? ~0ull : 0ull;
    const uint8_t *packed = reinterpret_cast<const uint8_t *>(
        pick3(m1, m2, (uint64_t)a.packed[0], (uint64_t)a.packed[1], (uint64_t)a.packed[2]));
    const int64_t M = (int64_t)pick3(m1, m2, (uint64_t)a.M[0], (uint64_t)a.M[1], (uint64_t)a.M[2]);
    return packed_scale(packed, M, a.K);
}

__device__ __forceinline__ TileRef resolve_tile(const GroupArgs &a, int64_t tile) {
    const uint64_t m1 = tile >= a.tiles_end[0] ? ~0ull : 0ull;
    const uint64_t m2 = tile >= a.tiles_end[1] ? ~0ull : 0ull;
    TileRef t;
    t.packed = reinterpret_cast<const uint8_t *>(
        pick3(m1, m2, (uint64_t)a.packed[0], (uint64_t)a.packed[1], (uint64_t)a.packed[2]));
    t.y = reinterpret_cast<void *>(
        pick3(m1, m2, (uint64_t)a.y[0], (uint64_t)a.y[1], (uint64_t)a.y[2]));
    t.M = (int64_t)pick3(m1, m2, (uint64_t)a.M[0], (uint64_t)a.M[1], (uint64_t)a.M[2]);
    t.mt = tile - (int64_t)pick3(m1, m2, 0ull, (uint64_t)a.tiles_end[0],
                                 (uint64_t)a.tiles_end[1]);
    t.proj = (int)(m1 & 1u) + (int)(m2 & 1u);
    return t;
}

}  // namespace bt
