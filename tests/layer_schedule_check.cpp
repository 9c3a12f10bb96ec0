// Host-side check of the one-launch block kernel's work schedule, against
// the library's own planner (bt::plan_layer_schedule) and the schedule view
// the kernel itself runs (bt::LayerSched).  For random block shapes and grid
// sizes, on 2-bit tiles (16 waves, K split 8: two tiles per iteration) and
// base-3 tiles (K split 4: four tiles per iteration):
//   - every row tile of the seven projections is taken by exactly one
//     sub-group of exactly one workgroup iteration;
//   - the waves of a sub-group split each tile's K blocks exactly (each block
//     once), every wave with at least one block;
//   - the closed-form slot count of each wave equals the walk over its
//     iterations (the kernel's cursors stop after that many slots, and every
//     wave of a workgroup runs the same iterations, each ending in a barrier);
//   - the prologue's per-wave input row tables (1 to 4 tokens) place every
//     input chunk at its own element, LDS byte and (group, token) key, and
//     the inputs a workgroup quantizes cover every tile it takes.
// Prints the schedule chosen for the 70B-class block; exit status 0 if every
// check passes.
#include <cstdio>
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <random>
#include <vector>

#include "layer.hpp"

namespace {

constexpr int kWaves = 16;

int g_fail = 0;
int g_modes[2] = {0, 0};
#define CHECK(c, ...)                                               \
    do {                                                            \
        if (!(c)) {                                                 \
            if (g_fail < 20) {                                      \
                std::printf("FAIL %s:%d ", __FILE__, __LINE__);     \
                std::printf(__VA_ARGS__);                           \
                std::printf("\n");                                  \
            }                                                       \
            ++g_fail;                                               \
        }                                                           \
    } while (0)

int group_of_tile(const bt::LayerArgs &a, int t) {
    int g = 0;
    while (g < 3 && t >= a.gend32[g]) ++g;
    return g;
}

// One block: M of q,k,v,o,gate,up,down and K of the four inputs.
void check(const int64_t M[7], const int64_t K[4], int G, bool b3) {
    const int P = b3 ? 4 : 8, tpw = kWaves / P;
    const uint8_t *w[7] = {};
    const void *x[4] = {};
    void *y[7] = {};
    bt::LayerArgs a = bt::make_layer_args(w, M, K, x, y, 1, BT_BF16, b3);
    bt::plan_layer_schedule(a, G, b3);
    ++g_modes[a.sched ? 1 : 0];
    const int total = a.tend32[6];
    std::vector<int> seen(total, 0);
    for (int wg = 0; wg < G; ++wg) {
        const bt::LayerSched ls(a, wg, G, tpw);
        // the inputs the workgroup's prologue quantizes cover every tile it
        // takes (exactly, under the two-class schedule)
        {
            uint32_t walk = 0;
            for (int it = 0; it < ls.nit; ++it)
                for (int s = 0; s < tpw; ++s) {
                    const int t = ls.tile_for(it, s);
                    if (t >= 0 && t < total) walk |= 1u << group_of_tile(a, t);
                }
            const uint32_t need =
                wg < bt::kLayerNeedWgs ? (a.need[wg / 8] >> (4 * (wg % 8))) & 0xFu : 0xFu;
            CHECK((walk & ~need) == 0, "wg %d reads inputs 0x%x, marked 0x%x", wg, walk, need);
            CHECK(!a.sched || wg >= bt::kLayerNeedWgs || walk == need,
                  "wg %d: two-class need 0x%x, walk 0x%x", wg, need, walk);
        }
        for (int wave = 0; wave < kWaves; ++wave) {
            const int kpart = wave % P, sub = wave / P;
            int walk = 0;
            for (int it = 0; it < ls.nit; ++it) {
                const int t = ls.tile_for(it, sub);
                if (t < total) walk += bt::LayerSched::nq(a, group_of_tile(a, t), kpart, P);
            }
            CHECK(walk == ls.slots(a, sub, kpart, P), "slots: wg %d wave %d walk %d formula %d",
                  wg, wave, walk, ls.slots(a, sub, kpart, P));
        }
        for (int it = 0; it < ls.nit; ++it) {
            for (int s = 0; s < tpw; ++s) {
                const int t = ls.tile_for(it, s);
                CHECK(t >= 0, "negative tile %d", t);
                if (t < 0 || t >= total) continue;
                ++seen[t];
                const int g = group_of_tile(a, t), qb = bt::LayerSched::blocks(a, g);
                std::vector<int> hit(qb, 0);
                for (int k = 0; k < P; ++k) {
                    CHECK(bt::LayerSched::nq(a, g, k, P) >= 1, "wave part %d has no block of tile %d", k, t);
                    for (int b = k; b < qb; b += P) ++hit[b];
                }
                for (int b = 0; b < qb; ++b) CHECK(hit[b] == 1, "block %d of tile %d", b, t);
            }
        }
    }
    for (int t = 0; t < total; ++t) CHECK(seen[t] == 1, "tile %d taken %d times", t, seen[t]);
}

// The prologue's per-wave row tables (bt::LayerWaveRows) for N tokens: every
// live chunk of every wave's span, located the way the kernel locates it
// (row #{r >= 1 : d >= st[r]}), addresses its own input element and LDS byte
// and carries its (group, token) key; a table with one row holds all of its
// span; dead spans hold nothing.
void check_rows(const int64_t M[7], const int64_t K[4], int64_t N) {
    if (!bt::layer_fusable(K, M, N, BT_BF16)) return;
    const uint8_t *w[7] = {};
    const void *x[4];
    void *y[7] = {};
    for (int g = 0; g < 4; ++g) x[g] = reinterpret_cast<const void *>((uintptr_t)(g + 1) << 36);
    const bt::LayerArgs a = bt::make_layer_args(w, M, K, x, y, N, BT_BF16, false);
    const int nt = N == 1 ? 1 : (N == 2 ? 2 : 4);
    int64_t units = 0;
    for (int g = 0; g < 4; ++g) units += N * K[g] / 8;
    for (int wv = 0; wv < bt::kLayerWaves; ++wv) {
        const bt::LayerWaveRows &t = a.wrows[wv];
        const int64_t u0 = (int64_t)wv * bt::kLayerSpan;
        const int64_t live = std::max<int64_t>(0, std::min<int64_t>(bt::kLayerSpan, units - u0));
        CHECK(t.nlive == live, "N %lld wave %d: nlive %d, want %lld", (long long)N, wv, t.nlive,
              (long long)live);
        CHECK(t.nrow >= 1 && t.nrow <= bt::kWaveRows, "wave %d: nrow %d", wv, t.nrow);
        for (int d = 0; d < live; ++d) {
            int r = 0;
            for (int k = 1; k < bt::kWaveRows; ++k) r += d >= t.st[k] ? 1 : 0;
            // the chunk's place by direct search
            int64_t u = u0 + d, g = 0;
            while (u >= N * K[g] / 8) u -= N * K[g] / 8, ++g;
            const int64_t j = u / (K[g] / 8), c = u % (K[g] / 8);
            const uintptr_t want_src = (uintptr_t)x[g] + (uintptr_t)(2 * (j * K[g] + 8 * c));
            const uintptr_t got_src = (uintptr_t)t.src[r] + (uintptr_t)(2 * 8 * d);
            CHECK(r < t.nrow, "N %lld wave %d chunk %d: row %d of %d", (long long)N, wv, d, r, t.nrow);
            CHECK(got_src == want_src, "N %lld wave %d chunk %d: source", (long long)N, wv, d);
            CHECK((int64_t)t.dst[r] + 8 * d == a.xoff[g] + j * K[g] + 8 * c,
                  "N %lld wave %d chunk %d: LDS byte", (long long)N, wv, d);
            CHECK(t.key[r] == g * nt + j, "N %lld wave %d chunk %d: key %d, want %lld",
                  (long long)N, wv, d, t.key[r], (long long)(g * nt + j));
        }
    }
    // the dead lanes' chunk: the last one of the last input
    CHECK((uintptr_t)a.xlast == (uintptr_t)x[3] + (uintptr_t)(2 * (N * K[3] - 8)), "xlast");
}

}  // namespace

int main(int argc, char **argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 2000;
    {
        const int64_t M[7] = {8192, 1024, 1024, 8192, 28672, 28672, 8192};
        const int64_t K[4] = {8192, 8192, 8192, 28672};
        check(M, K, 256, false);
        check(M, K, 256, true);
        for (int n = 1; n <= 4; ++n) check_rows(M, K, n);
        const int64_t M2[7] = {2560, 640, 640, 2560, 6912, 6912, 2560};
        const int64_t K2[4] = {2560, 2560, 2560, 6912};
        for (int n = 1; n <= 4; ++n) check_rows(M2, K2, n);
        const int64_t M3[7] = {2048, 2048, 2048, 2048, 2048, 2048, 2048};
        const int64_t K3[4] = {2048, 2048, 2048, 2048};
        for (int n = 1; n <= 4; ++n) check_rows(M3, K3, n);
        const uint8_t *w[7] = {};
        const void *x[4] = {};
        void *y[7] = {};
        bt::LayerArgs a = bt::make_layer_args(w, M, K, x, y, 1, BT_BF16, false);
        bt::plan_layer_schedule(a, 256, false);
        std::printf("70B-class block, 256 workgroups: sched %d, n0 %d, heavy %d/%d, light groups %d/%d\n",
                    a.sched, a.n0, a.heavy[0], a.heavy[1], a.scount[0], a.scount[1]);
        int hist[16] = {};
        for (int wg = 0; wg < 256; ++wg) ++hist[(a.need[wg / 8] >> (4 * (wg % 8))) & 0xFu];
        std::printf("inputs read per workgroup (mask: workgroups):");
        for (int m = 0; m < 16; ++m)
            if (hist[m]) std::printf(" 0x%x: %d", m, hist[m]);
        std::printf("\n");
    }
    std::mt19937 rng(20241021);
    auto pick = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    for (int c = 0; c < cases && g_fail == 0; ++c) {
        const bool b3 = pick(0, 3) == 0;
        const int unit = b3 ? 1024 : 256, minb = b3 ? 4 : 8;
        int64_t M[7], K[4];
        for (int g = 0; g < 4; ++g) K[g] = unit * (int64_t)pick(minb, minb * 6);
        if (pick(0, 2)) {
            // the usual block: q, k, v, o, gate, up of one width, a wider down
            // projection (two kinds of tile groups)
            K[0] = K[1] = K[2] = unit * (int64_t)pick(minb, minb * 5);
            K[3] = K[0] + unit * (int64_t)pick(1, minb * 12);
        }
        for (int p = 0; p < 7; ++p) M[p] = 16 * (int64_t)pick(1, 600);
        check(M, K, pick(1, 300), b3);
        if (!b3) check_rows(M, K, pick(1, 4));
    }
    std::printf("%s after %d random blocks (schedules: %d striding, %d two-class)\n",
                g_fail ? "FAILED" : "ok", cases, g_modes[0], g_modes[1]);
    return g_fail ? 1 : 0;
}
