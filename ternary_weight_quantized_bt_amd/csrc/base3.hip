// base3.hip -- the denser base-3 weight format "B3T1024": 64 ternary weights
// in 13 bytes (1.625 bits per weight), its packing, unpacking and decode
// product.
//
// [IK] "ik_llama.cpp 运行 BitNet b1.58 2B 模型实战…", sections 5.2, 5.3 and 6:
// a 1.625-bit ternary format over blocks of 64 weights, decoded with integer
// arithmetic rather than 2-bit masks.  The pages give the density and the
// block, not the bytes; the encoding and the tile layout are this library's
// (libternary.h defines both):
//   codes c = w + 1; byte j < 12 of a block = c[4j] + 3 c[4j+1] + 9 c[4j+2]
//   + 27 c[4j+3] + 81 c[48+j] (0..242); byte 12 = c[60] + 3 c[61] + 9 c[62]
//   + 27 c[63] (0..80).
//   Tile = 16 rows x 1024 columns = 3328 bytes.  Lane l = r + 16 s holds row
//   r, columns 256 s .. 256 s + 255 (blocks b = 0..3) in 13 words: words
//   3b .. 3b+2 are bytes 0..11 of block b, word 12 byte b is byte 12 of block
//   b; words 0..11 sit in three 16-byte chunks at 16 (64 i + l) (a wave reads
//   each chunk row with one coalesced 128-bit load), word 12 at 3072 + 4 l.
//
// The decode (an LDS table of the four low digits of every byte value, the
// fifth digits merged with byte permutes) is in base3.hpp, shared with the
// per-layer kernel.

#include "base3.hpp"
#include "internal.hpp"

namespace bt {

namespace {

// ---------------------------------------------------------------- packing --

constexpr int kB3PackThreads = 256;

// Code (0, 1, 2) of a signed byte; values outside {-1, 0, 1} are clamped
// to the nearest state and counted.
__device__ __forceinline__ uint32_t code_of(int8_t v, int &bad) {
    int x = v;
    if (x < -1) { x = -1; ++bad; }
    if (x > 1) { x = 1; ++bad; }
    return (uint32_t)(x + 1);
}

// One thread per (tile, lane): reads the lane's 256 weights (row r, columns
// 256 s ..), writes its three 16-byte chunks and its last word.
__global__ __launch_bounds__(kB3PackThreads)
void b3_pack_kernel(const int8_t *__restrict__ w, int64_t M, int64_t K, float scale,
                    uint8_t *__restrict__ packed, int32_t *__restrict__ invalid) {
    const int64_t qc = K / kB3Cols;
    const int64_t nruns = (M / kTileRows) * qc * kWave;
    const int64_t run = (int64_t)blockIdx.x * kB3PackThreads + threadIdx.x;
    int bad = 0;
    if (run < nruns) {
        const int64_t tile = run / kWave;
        const int lane = (int)(run % kWave);
        const int64_t mt = tile / qc, q = tile % qc;
        const int r = lane % 16, s = lane / 16;
        const int8_t *src = w + (mt * kTileRows + r) * K + q * kB3Cols + 256 * s;
        uint32_t words[13];
        uint32_t last = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t c[64];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src + 64 * b + 16 * u);
                const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    c[16 * u + e] = code_of((int8_t)(in[e / 4] >> (8 * (e % 4))), bad);
            }
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                uint32_t word = 0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int j = 4 * i + t;
                    const uint32_t byte = c[4 * j] + 3 * c[4 * j + 1] + 9 * c[4 * j + 2] +
                                          27 * c[4 * j + 3] + 81 * c[48 + j];
                    word |= byte << (8 * t);
                }
                words[3 * b + i] = word;
            }
            last |= (c[60] + 3 * c[61] + 9 * c[62] + 27 * c[63]) << (8 * b);
        }
        words[12] = last;
        uint8_t *t0 = packed + tile * kB3TileBytes;
#pragma unroll
        for (int i = 0; i < 3; ++i)
            reinterpret_cast<v4u *>(t0)[64 * i + lane] =
                v4u{words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]};
        reinterpret_cast<uint32_t *>(t0 + 3072)[lane] = last;
    }
    if (invalid != nullptr) {
        const int total = wave_sum(bad);
        if ((threadIdx.x % kWave) == 0 && total != 0) atomicAdd(invalid, total);
    }
    // Tail: the scale, then zeros up to 256 bytes.
    if (blockIdx.x == 0 && threadIdx.x < BT_TAIL_BYTES / 4) {
        uint32_t *tail = reinterpret_cast<uint32_t *>(packed + b3_code_bytes(M, K));
        tail[threadIdx.x] = threadIdx.x == 0 ? __float_as_uint(scale) : 0u;
    }
}

// Inverse of b3_pack_kernel: w = code - 1.
__global__ __launch_bounds__(kB3PackThreads)
void b3_unpack_kernel(const uint8_t *__restrict__ packed, int64_t M, int64_t K,
                      int8_t *__restrict__ w) {
    const int64_t qc = K / kB3Cols;
    const int64_t nruns = (M / kTileRows) * qc * kWave;
    const int64_t run = (int64_t)blockIdx.x * kB3PackThreads + threadIdx.x;
    if (run >= nruns) return;
    const int64_t tile = run / kWave;
    const int lane = (int)(run % kWave);
    const int64_t mt = tile / qc, q = tile % qc;
    const int r = lane % 16, s = lane / 16;
    const uint8_t *t0 = packed + tile * kB3TileBytes;
    uint32_t words[13];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const v4u v = reinterpret_cast<const v4u *>(t0)[64 * i + lane];
        words[4 * i] = v.x;
        words[4 * i + 1] = v.y;
        words[4 * i + 2] = v.z;
        words[4 * i + 3] = v.w;
    }
    words[12] = reinterpret_cast<const uint32_t *>(t0 + 3072)[lane];
    int8_t *dst = w + (mt * kTileRows + r) * K + q * kB3Cols + 256 * s;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t out[16];
        uint32_t fifth[3] = {0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 12; ++j) {
            const uint32_t v = (words[3 * b + j / 4] >> (8 * (j % 4))) & 0xFFu;
            out[j] = low_digits(v);
            fifth[j / 4] |= (v / 81) << (8 * (j % 4));
        }
#pragma unroll
        for (int g = 0; g < 3; ++g) out[12 + g] = fifth[g];
        out[15] = low_digits((words[12] >> (8 * b)) & 0xFFu);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // bytewise c - 1 for c in 0..2: (c + 128 - 1) ^ 128 in every
                // byte, no borrow between bytes
                const uint32_t c = out[4 * u + e];
                o[e] = ((c | 0x80808080u) - 0x01010101u) ^ 0x80808080u;
            }
            *reinterpret_cast<uint4 *>(dst + 64 * b + 16 * u) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// ----------------------------------------------------------- decode GEMV --

struct B3Args {
    const uint8_t *packed;
    int64_t M, K;
    const int8_t *xq;     // [N, K] codes of this launch's tokens
    const float *xs;      // [N]
    const int32_t *xsum;  // [N]
    int64_t N;            // tokens of this launch, 1..NT
    void *y;              // [N, M] outputs of this launch's tokens
    int ydt;
};

// Decode product over B3 tiles.  Persistent grid: each workgroup builds the
// table and stages the activations (LDSX) in LDS, then walks the 16-row
// tiles with a stride of the grid.  Its WAVES waves split K into P contiguous
// runs of 1024-column tiles (TPW = WAVES / P row tiles per iteration); each
// wave keeps RING tile slots in flight (non-temporal loads), across tile
// boundaries.  Row sums are reduced over the four lanes of a row (xor
// shuffles), then over the P waves through LDS (one barrier per iteration),
// and dequantized.
template <int NT, bool LDSX, int WAVES, int P, int RING>
__global__ __launch_bounds__(WAVES * kWave)
void b3_gemv_kernel(B3Args a) {
    static_assert(WAVES % P == 0, "K split must divide the waves");
    constexpr int kThreads = WAVES * kWave;
    constexpr int TPW = WAVES / P;
    extern __shared__ __attribute__((aligned(16))) uint8_t b3_smem[];
    __shared__ int red[P > 1 ? 2 : 1][P > 1 ? WAVES : 1][NT][16];
    __shared__ float s_factor[NT];
    __shared__ int s_xsum[NT];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t K = a.K, qc = K / kB3Cols, mtiles = a.M / kTileRows;
    const int nvalid = (int)min((int64_t)NT, a.N);
    const int kpart = wave % P, sub = wave / P;
    const int64_t c0 = qc * kpart / P, c1 = qc * (kpart + 1) / P;
    const int64_t nq = c1 - c0;  // tiles of this wave per row tile (may be 0)
    const int64_t ngroups = (mtiles + TPW - 1) / TPW;
    const int64_t nit = (ngroups - blockIdx.x + gridDim.x - 1) / gridDim.x;
    auto tile_of = [&](int64_t it) { return (blockIdx.x + it * gridDim.x) * TPW + sub; };
    const bool has_work = nq > 0 && tile_of(0) < mtiles;
    const int64_t nslots = has_work ? nit * nq : 0;
    auto tile_ptr = [&](int64_t mt, int64_t c) { return a.packed + (mt * qc + c) * kB3TileBytes; };

    // Load cursor; past the last valid slot it stays put, so every ring load
    // is unconditional (a harmless reload).
    int64_t li = 0, lit = 0, lc = c0;
    bool lvalid = has_work;
    const uint8_t *lp = has_work ? tile_ptr(tile_of(0), c0) : a.packed;
    auto advance_load = [&]() {
        if (++li >= nslots || !lvalid) return;
        if (++lc < c1) {
            lp += kB3TileBytes;
            return;
        }
        lc = c0;
        ++lit;
        const int64_t t = tile_of(lit);
        if (t < mtiles) lp = tile_ptr(t, c0);
        else lvalid = false;
    };

    B3Slot ring[RING];
    if (has_work) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            ring[d] = load_slot<true>(lp, lane);
            advance_load();
        }
    }

    // ---- prologue: the table, the activations, the per-token constants ----
    uint8_t *tab = b3_smem;
    b3_build_table(tab, (int)threadIdx.x, kThreads);
    const int8_t *xsrc = a.xq;
    if (LDSX) {
        int8_t *xl = reinterpret_cast<int8_t *>(b3_smem + kB3TabBytes);
        const int64_t n16 = nvalid * K / 16;
        for (int64_t e = threadIdx.x; e < n16; e += kThreads)
            reinterpret_cast<v4u *>(xl)[e] = to_global(reinterpret_cast<const v4u *>(a.xq))[e];
        xsrc = xl;
    }
    if ((int)threadIdx.x < nvalid) {
        const float sw = *to_global(reinterpret_cast<const float *>(a.packed + b3_code_bytes(a.M, K)));
        s_xsum[threadIdx.x] = a.xsum[threadIdx.x];
        s_factor[threadIdx.x] = token_factor(sw, a.xs[threadIdx.x]);
    }
    __syncthreads();
    const uint32_t l8 = 8u * (uint32_t)(lane % kB3Copies);
    const int8_t *xb = xsrc + 256 * (lane / 16);

    int buf = 0;
    int acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = 0;
    auto iter_done = [&](int64_t it) {
        int v[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            v[n] = acc[n];
            v[n] += __shfl_xor(v[n], 16, kWave);
            v[n] += __shfl_xor(v[n], 32, kWave);
            acc[n] = 0;
        }
        if (P == 1) {
            const int64_t mt = tile_of(it);
            if (lane < 16 && mt < mtiles) {
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if (n >= nvalid) break;
                    store_out(a.y, a.ydt, n * a.M + mt * kTileRows + lane, v[n] - s_xsum[n],
                              s_factor[n]);
                }
            }
        } else {
            if (lane < 16) {
#pragma unroll
                for (int n = 0; n < NT; ++n) red[buf][wave][n][lane] = v[n];
            }
            __syncthreads();
            if (threadIdx.x < TPW * 16 * NT) {
                const int s = threadIdx.x / (16 * NT);
                const int n = (threadIdx.x / 16) % NT, r = threadIdx.x % 16;
                const int64_t mt = (blockIdx.x + it * gridDim.x) * TPW + s;
                if (n < nvalid && mt < mtiles) {
                    int t = 0;
#pragma unroll
                    for (int p = 0; p < P; ++p) t += red[buf][s * P + p][n][r];
                    store_out(a.y, a.ydt, n * a.M + mt * kTileRows + r, t - s_xsum[n],
                              s_factor[n]);
                }
            }
            buf ^= 1;
        }
    };

    if (!has_work) {
        if (P > 1)
            for (int64_t it = 0; it < nit; ++it) iter_done(it);
        return;
    }
    int64_t cc = c0, cit = 0;  // compute cursor: tile column, iteration
    for (int64_t base = 0; base < nslots; base += RING) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
            const int64_t i = base + d;
            const B3Slot cur = ring[d];
            ring[d] = load_slot<true>(lp, lane);
            advance_load();
            if (i < nslots) {
                b3_dot<NT>(cur, tab, l8, xb + cc * kB3Cols, K, nvalid, acc);
                if (++cc == c1) {
                    iter_done(cit);
                    cc = c0;
                    ++cit;
                }
            }
        }
    }
}

constexpr int kB3Ring = 2;

// Static LDS of b3_gemv_kernel (the reduction buffers, per-token constants).
constexpr size_t b3_static_lds(int nt) { return 2 * 16 * nt * 16 * 4 + 64; }

int max_lds_per_cu() { return 160 * 1024; }

int max_lds_per_block() {
    static int lds[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
    if (lds[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess || v <= 0)
            v = 64 * 1024;
        lds[dev] = v;
    }
    return lds[dev];
}

template <int NT, bool LDSX, int WAVES, int P>
hipError_t launch_b3_p(const B3Args &a, size_t shmem, hipStream_t s) {
    constexpr int TPW = WAVES / P;
    auto kern = b3_gemv_kernel<NT, LDSX, WAVES, P, kB3Ring>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)shmem);
    if (e != hipSuccess) return e;
    const int64_t groups = (a.M / kTileRows + TPW - 1) / TPW;
    const int per_cu = (int)max((size_t)1, min((size_t)2, (size_t)max_lds_per_cu() /
                                                          (shmem + b3_static_lds(NT))));
    const int64_t grid = min(groups, (int64_t)device_cus() * per_cu);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * kWave), shmem, s, a);
    return hipGetLastError();
}

// Launch shape.  Every iteration of a workgroup ends in a cross-wave
// reduction and a barrier that cost about as much as streaming two or three
// tiles, so iterations should be few and long:
//   - enough row tiles to give three quarters of the compute units a group
//     of 8, and LDS for two workgroups per unit: 8 waves that each own a
//     whole row tile (no K split, no barrier);
//   - otherwise 16 waves (8 for four tokens: registers), split along K into
//     the fewest parts P that still give every compute unit a workgroup, at
//     most 8 and at most one part per tile column.
template <int NT, bool LDSX>
hipError_t launch_b3_x(const B3Args &a, size_t shmem, hipStream_t s) {
    const int64_t mtiles = a.M / kTileRows, qc = a.K / kB3Cols;
    const int64_t cus = device_cus();
    const bool two_per_cu = 2 * (shmem + b3_static_lds(NT)) <= (size_t)max_lds_per_cu();
    if (two_per_cu && (mtiles + 7) / 8 * 4 >= 3 * cus)
        return launch_b3_p<NT, LDSX, 8, 1>(a, shmem, s);
    constexpr int W = NT == 4 ? 8 : 16;
    int pmax = 1;
    while (pmax < 8 && 2 * pmax <= qc) pmax *= 2;
    int P = 1;
    while (P < pmax && (mtiles + W / P - 1) / (W / P) < cus) P *= 2;
    switch (P) {
        case 1: return launch_b3_p<NT, LDSX, W, 1>(a, shmem, s);
        case 2: return launch_b3_p<NT, LDSX, W, 2>(a, shmem, s);
        case 4: return launch_b3_p<NT, LDSX, W, 4>(a, shmem, s);
        default: return launch_b3_p<NT, LDSX, W, 8>(a, shmem, s);
    }
}

template <int NT>
hipError_t launch_b3_nt(const B3Args &a, hipStream_t s) {
    const size_t with_x = (size_t)kB3TabBytes + (size_t)(NT * a.K);
    if ((int64_t)(with_x + b3_static_lds(NT)) <= (int64_t)max_lds_per_block())
        return launch_b3_x<NT, true>(a, with_x, s);
    return launch_b3_x<NT, false>(a, (size_t)kB3TabBytes, s);
}

}  // namespace

hipError_t launch_b3_pack(const int8_t *w, int64_t M, int64_t K, float scale, uint8_t *packed,
                          int32_t *invalid, hipStream_t s) {
    const int64_t nruns = (M / kTileRows) * (K / kB3Cols) * kWave;
    const int64_t blocks = (nruns + kB3PackThreads - 1) / kB3PackThreads;
    hipLaunchKernelGGL(b3_pack_kernel, dim3((unsigned)blocks), dim3(kB3PackThreads), 0, s, w, M,
                       K, scale, packed, invalid);
    return hipGetLastError();
}

hipError_t launch_b3_unpack(const uint8_t *packed, int64_t M, int64_t K, int8_t *w,
                            hipStream_t s) {
    const int64_t nruns = (M / kTileRows) * (K / kB3Cols) * kWave;
    const int64_t blocks = (nruns + kB3PackThreads - 1) / kB3PackThreads;
    hipLaunchKernelGGL(b3_unpack_kernel, dim3((unsigned)blocks), dim3(kB3PackThreads), 0, s,
                       packed, M, K, w);
    return hipGetLastError();
}

// Tokens in passes of up to four (each pass streams the weights once).
hipError_t launch_b3_gemv(const uint8_t *packed, int64_t M, int64_t K, const int8_t *xq,
                          const float *xs, const int32_t *xsum, int64_t N, void *y,
                          bt_dtype ydt, hipStream_t s) {
    const int64_t esize = ydt == BT_BF16 ? 2 : 4;
    for (int64_t n0 = 0; n0 < N; n0 += 4) {
        const int64_t nt = min((int64_t)4, N - n0);
        const B3Args a{packed, M, K, xq + n0 * K, xs + n0, xsum + n0, nt,
                       static_cast<uint8_t *>(y) + n0 * M * esize, (int)ydt};
        hipError_t e;
        if (nt == 1) e = launch_b3_nt<1>(a, s);
        else if (nt == 2) e = launch_b3_nt<2>(a, s);
        else e = launch_b3_nt<4>(a, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bt
