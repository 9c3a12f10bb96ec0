// wquant.hip -- float -> ternary weight quantizer, straight into the packed
// T16Q256 layout.
//
// "LLM Quantization Paradigms: FP8, AWQ, EXL2 & BitNet b1.58 in 2026",
// section 5 ("The Mathematics of BitNet b1.58"): the AbsMean quantizer,
// gamma = mean |W| over the whole tensor and W~ = RoundClip(W / (gamma +
// eps), -1, 1) with RoundClip(x) = max(-1, min(1, round(x))).  "How BitNet's
// 1-Bit (I2_S) Quantization Works Compared to Standard LLM Quantization",
// "Per-Tensor Scaling Strategy": the I2_S per-tensor scale is max|w|.
//
// Definitions this file implements (libternary.h states them for callers):
//   s = max|W|, or mean|W| = (exact sum of |W|) / (M*K) rounded once to the
//       nearest float32 (ties to even): no summation order can change it;
//   d = float32(s + eps), the divisor and the scale stored in the tail;
//   code = RoundClip(float32(W / d)) + 1, round half to even, 0/0 -> 0.
//
// Five launches on the caller's stream:
//   1. clear the state block (a fill kernel, so the sequence can be captured
//      in a graph);
//   2. max of the |W| bit patterns (an unsigned compare orders non-negative
//      finite floats), one atomic per workgroup;
//   3. (AbsMean only) the exact sum.  With E the exponent of the max, a
//      value m * 2^(e-150) (m the 24-bit significand, e the biased exponent,
//      at least 1) with E - e < 32 adds m << (31 - (E - e)) -- at most 55
//      bits -- to window 0, split into its two 32-bit halves so that no
//      64-bit accumulator can overflow for up to 2^31 elements; E - e in
//      [32, 64) goes the same way to window 1; anything smaller (rare for
//      weights) adds m to a per-exponent bin in LDS.  All sums are integers,
//      so atomics in any order give the same totals;
//   4. one thread turns the integers into s (a 384-bit sum divided by M*K
//      and rounded), d, and a float32 threshold t: since float32 division is
//      correctly rounded and rounding is monotone, round(W / d) is +-1
//      exactly when |W| > d * (0.5 + 2^-25) (the midpoint above 0.5); that
//      product is exact in float64 and t is the smallest float32 above it,
//      so the packing kernel decides each code with one integer compare of
//      |W|'s bits against t's;
//   5. pack: one thread per 16-byte slot, as the int8 packer does, plus the
//      tail (d, then zeros).

#include "common.hpp"
#include "internal.hpp"
#include "quant.hpp"

namespace bt {

namespace {

constexpr int kWqThreads = 256;
constexpr int kWqWaves = kWqThreads / kWave;

// Device state of one quantization (lives in the caller's workspace).
struct WqState {
    uint32_t max_bits;       // max |W| as float32 bits
    uint32_t thr_bits;       // code threshold (see the header)
    float s, d;              // statistic and divisor
    unsigned long long win[4];   // window 0 low / high halves, window 1 low / high
    unsigned long long bins[256];  // significand sums of small values per exponent
};
static_assert(sizeof(WqState) <= BT_WQ_WORKSPACE_BYTES, "workspace size");

// float32 bits of 8 consecutive elements.
__device__ __forceinline__ void load_bits8(const float *p, uint32_t (&u)[8]) {
    const v4u a = *to_global(reinterpret_cast<const v4u *>(p));
    const v4u b = *to_global(reinterpret_cast<const v4u *>(p) + 1);
    u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w;
    u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
}
__device__ __forceinline__ void load_bits8(const uint16_t *p, uint32_t (&u)[8]) {
    const v4u a = *to_global(reinterpret_cast<const v4u *>(p));
    const uint32_t h[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // bfloat16 -> float32 bits (exact)
        u[2 * i] = h[i] << 16;
        u[2 * i + 1] = h[i] & 0xFFFF0000u;
    }
}

__global__ void wq_clear_kernel(WqState *st) {
    uint32_t *p = reinterpret_cast<uint32_t *>(st);
    for (int i = threadIdx.x; i < (int)(sizeof(WqState) / 4); i += blockDim.x) p[i] = 0u;
}

template <typename T>
__global__ __launch_bounds__(kWqThreads)
void wq_max_kernel(const T *__restrict__ w, int64_t chunks, WqState *st) {
    __shared__ uint32_t red[kWqWaves];
    uint32_t m = 0;
    for (int64_t c = (int64_t)blockIdx.x * kWqThreads + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * kWqThreads) {
        uint32_t u[8];
        load_bits8(w + 8 * c, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = max(m, u[i] & 0x7FFFFFFFu);
    }
    m = wave_reduce<true>(m);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = red[0];
#pragma unroll
        for (int i = 1; i < kWqWaves; ++i) v = max(v, red[i]);
        atomicMax(&st->max_bits, v);
    }
}

// Per-thread window sums (see the header): window 0 low / high halves,
// window 1 low / high halves, in the order of WqState::win.
struct WinAcc {
    unsigned long long v[4];
};

// Adds |bits| to the windows; returns true (with the exponent e and the
// significand m) when the value is too small for them and goes to a bin.
__host__ __device__ inline bool accumulate(uint32_t bits, uint32_t E, WinAcc &acc,
                                           uint32_t &e, uint32_t &m) {
    const uint32_t a = bits & 0x7FFFFFFFu;
    const uint32_t ef = a >> 23;
    m = (a & 0x7FFFFFu) | (ef != 0u ? 0x800000u : 0u);
    e = ef > 1u ? ef : 1u;
    const uint32_t dd = E - e;  // a <= max, so e <= E
    const uint64_t v0 = dd < 32u ? (uint64_t)m << (31u - dd) : 0ull;
    const uint64_t v1 = dd - 32u < 32u ? (uint64_t)m << (63u - dd) : 0ull;
    acc.v[0] += (uint32_t)v0;
    acc.v[1] += (uint32_t)(v0 >> 32);
    acc.v[2] += (uint32_t)v1;
    acc.v[3] += (uint32_t)(v1 >> 32);
    return dd >= 64u && m != 0u;
}

__device__ __forceinline__ unsigned long long wave_sum64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

template <typename T>
__global__ __launch_bounds__(kWqThreads)
void wq_sum_kernel(const T *__restrict__ w, int64_t chunks, WqState *st) {
    __shared__ unsigned long long bins[256];
    __shared__ unsigned long long red[4][kWqWaves];
    for (int i = threadIdx.x; i < 256; i += kWqThreads) bins[i] = 0;
    __syncthreads();
    // exponent field of the max, at least 1 (subnormals share exponent 1)
    const uint32_t E = max(__builtin_amdgcn_readfirstlane(st->max_bits) >> 23, 1u);
    WinAcc acc{};
    for (int64_t c = (int64_t)blockIdx.x * kWqThreads + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * kWqThreads) {
        uint32_t u[8];
        load_bits8(w + 8 * c, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t e, m;
            if (accumulate(u[i], E, acc, e, m)) atomicAdd(&bins[e], (unsigned long long)m);
        }
    }
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned long long v = wave_sum64(acc.v[i]);
        if (lane == 0) red[i][wave] = v;
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        unsigned long long v = 0;
#pragma unroll
        for (int i = 0; i < kWqWaves; ++i) v += red[threadIdx.x][i];
        if (v != 0) atomicAdd(&st->win[threadIdx.x], v);
    }
    for (int i = threadIdx.x; i < 256; i += kWqThreads)
        if (bins[i] != 0) atomicAdd(&st->bins[i], bins[i]);
}

// 384-bit unsigned integer, 32-bit limbs, least significant first.
constexpr int kLimbs = 12;

__host__ __device__ inline void big_add(uint32_t (&x)[kLimbs], unsigned long long v, int shift) {
    int j = shift >> 5;
    const int r = shift & 31;
    // v << r spans up to three limbs
    unsigned long long lo = v << r;
    unsigned long long hi = r ? (v >> (64 - r)) : 0ull;
    const uint32_t part[3] = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi};
    unsigned long long carry = 0;
    for (int k = 0; j + k < kLimbs; ++k) {
        const unsigned long long add = (k < 3 ? part[k] : 0u);
        if (k >= 3 && carry == 0) break;
        const unsigned long long t = (unsigned long long)x[j + k] + add + carry;
        x[j + k] = (uint32_t)t;
        carry = t >> 32;
    }
}

__host__ __device__ inline int big_bits(const uint32_t (&x)[kLimbs]) {  // bit length
    for (int j = kLimbs - 1; j >= 0; --j)
        if (x[j] != 0u) return 32 * j + 32 - __builtin_clz(x[j]);
    return 0;
}

__host__ __device__ inline uint32_t big_bit(const uint32_t (&x)[kLimbs], int i) {
    return (i >= 0 && i < 32 * kLimbs) ? (x[i >> 5] >> (i & 31)) & 1u : 0u;
}

__host__ __device__ inline bool big_any_below(const uint32_t (&x)[kLimbs], int i) {  // bits [0, i)
    for (int j = 0; j < kLimbs && 32 * j < i; ++j) {
        const int n = i - 32 * j < 32 ? i - 32 * j : 32;
        const uint32_t mask = n == 32 ? 0xFFFFFFFFu : ((1u << n) - 1u);
        if (x[j] & mask) return true;
    }
    return false;
}

// The mean, rounded once: sum = X * 2^B, mean = X / n * 2^B.
__host__ __device__ inline float exact_mean(const WqState *st, int64_t n) {
    const int E = st->max_bits >> 23 > 1u ? (int)(st->max_bits >> 23) : 1;
    const int B = E - 213 < -149 ? E - 213 : -149;  // unit of the least significant bit of X
    uint32_t x[kLimbs] = {};
    big_add(x, st->win[0], E - 181 - B);
    big_add(x, st->win[1], E - 181 + 32 - B);
    big_add(x, st->win[2], E - 213 - B);
    big_add(x, st->win[3], E - 213 + 32 - B);
    for (int e = 1; e < 256; ++e)
        if (st->bins[e] != 0) big_add(x, st->bins[e], e - 150 - B);
    // Q = X / n, R = X % n (n < 2^32)
    const unsigned long long nn = (unsigned long long)n;
    unsigned long long rem = 0;
    for (int j = kLimbs - 1; j >= 0; --j) {
        const unsigned long long cur = (rem << 32) | x[j];
        x[j] = (uint32_t)(cur / nn);
        rem = cur % nn;
    }
    // keep 24 significant bits, or the bits down to 2^-149
    const int p = big_bits(x) - 1;                 // -1 when Q == 0
    const int q = p + B - 23 > -149 ? p + B - 23 : -149;  // exponent of the last kept bit
    const int k = q - B;                            // bits of Q dropped (B <= -149 <= q)
    uint32_t m = 0;
    for (int i = 0; i < 25; ++i) m |= big_bit(x, k + i) << i;
    bool up;
    if (k == 0) {
        up = 2 * rem > nn || (2 * rem == nn && (m & 1u));
    } else {
        const bool half = big_bit(x, k - 1) != 0u;
        const bool sticky = big_any_below(x, k - 1) || rem != 0;
        up = half && (sticky || (m & 1u));
    }
    m += up ? 1u : 0u;
    return __builtin_ldexpf((float)m, q);  // m <= 2^24: exact
}

// Bits of the smallest float32 above d * (0.5 + 2^-25), a product that is
// exact in float64 (24 + 25 significant bits).
__host__ __device__ inline uint32_t code_threshold(float d) {
    const double t = (double)d * (0.5 + 0x1p-25);
    const float t32 = (float)t;  // round to nearest
    uint32_t tb;
    __builtin_memcpy(&tb, &t32, 4);
    return (double)t32 <= t ? tb + 1u : tb;
}

__global__ void wq_finalize_kernel(WqState *st, int64_t n, int mode, float eps, float *stats) {
    if (threadIdx.x != 0) return;
    const float s = mode == BT_WSCALE_ABSMAX ? __uint_as_float(st->max_bits) : exact_mean(st, n);
    const float d = __fadd_rn(s, eps);
    st->s = s;
    st->d = d;
    st->thr_bits = code_threshold(d);
    if (stats != nullptr) {
        stats[0] = s;
        stats[1] = d;
    }
}

// One 32-bit packed word from 16 consecutive elements (bits of float32):
// column c goes to byte c % 4, bits 6 - 2 * (c / 4).
__device__ __forceinline__ uint32_t ternary_word(const uint32_t (&u)[16], uint32_t thr) {
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const uint32_t a = u[c] & 0x7FFFFFFFu;
        const uint32_t code = a >= thr ? ((u[c] >> 31) ? 0u : 2u) : 1u;
        word |= code << (8 * (c & 3) + 6 - 2 * (c >> 2));
    }
    return word;
}

template <typename T>
__global__ __launch_bounds__(kWqThreads)
void wq_pack_kernel(const T *__restrict__ w, int64_t M, int64_t K, const WqState *st,
                    uint8_t *__restrict__ packed) {
    const int64_t qb = K / kTileCols;
    const int64_t nslots = (M / kTileRows) * qb * kWave;
    const int64_t slot = (int64_t)blockIdx.x * kWqThreads + threadIdx.x;
    const uint32_t thr = __builtin_amdgcn_readfirstlane(st->thr_bits);
    if (slot < nslots) {
        const int64_t tile = slot / kWave;
        const int lane = (int)(slot % kWave);
        const int64_t mt = tile / qb, q = tile % qb;
        const int r = lane % 16, h = lane / 16;
        const T *src = w + (mt * kTileRows + r) * K + q * kTileCols + 16 * h;
        uint32_t out[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t u[16];
            uint32_t a[8], b[8];
            load_bits8(src + 64 * t, a);
            load_bits8(src + 64 * t + 8, b);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u[i] = a[i];
                u[8 + i] = b[i];
            }
            out[t] = ternary_word(u, thr);
        }
        *to_global(reinterpret_cast<v4u *>(packed) + slot) = v4u{out[0], out[1], out[2], out[3]};
    }
    if (blockIdx.x == 0 && threadIdx.x < BT_TAIL_BYTES / 4) {
        uint32_t *tail = reinterpret_cast<uint32_t *>(packed + M * K / 4);
        tail[threadIdx.x] = threadIdx.x == 0 ? __float_as_uint(st->d) : 0u;
    }
}

template <typename T>
hipError_t launch_wq_t(const T *w, int64_t M, int64_t K, int mode, float eps,
                       uint8_t *packed, float *stats, WqState *st, hipStream_t s) {
    const int64_t n = M * K, chunks = n / 8;
    const int64_t want = (chunks + kWqThreads - 1) / kWqThreads;
    const int64_t cap = (int64_t)device_cus() * 8;
    const unsigned grid = (unsigned)(want < cap ? want : cap);
    hipLaunchKernelGGL(wq_clear_kernel, dim3(1), dim3(kWqThreads), 0, s, st);
    hipLaunchKernelGGL((wq_max_kernel<T>), dim3(grid), dim3(kWqThreads), 0, s, w, chunks, st);
    if (mode == BT_WSCALE_ABSMEAN)
        hipLaunchKernelGGL((wq_sum_kernel<T>), dim3(grid), dim3(kWqThreads), 0, s, w, chunks, st);
    hipLaunchKernelGGL(wq_finalize_kernel, dim3(1), dim3(kWave), 0, s, st, n, mode, eps, stats);
    const int64_t nslots = (M / kTileRows) * (K / kTileCols) * kWave;
    const int64_t blocks = (nslots + kWqThreads - 1) / kWqThreads;
    hipLaunchKernelGGL((wq_pack_kernel<T>), dim3((unsigned)blocks), dim3(kWqThreads), 0, s,
                       w, M, K, st, packed);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_weights(const void *w, bt_dtype wdt, int64_t M, int64_t K, int mode,
                                   float eps, uint8_t *packed, float *stats, void *workspace,
                                   hipStream_t s) {
    WqState *st = static_cast<WqState *>(workspace);
    if (wdt == BT_F32)
        return launch_wq_t(static_cast<const float *>(w), M, K, mode, eps, packed, stats, st, s);
    return launch_wq_t(static_cast<const uint16_t *>(w), M, K, mode, eps, packed, stats, st, s);
}

}  // namespace bt
