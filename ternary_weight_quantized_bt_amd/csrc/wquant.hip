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
//      bits -- to window 0, whose 64-bit sums are folded into 32-bit halves
//      often enough that nothing can overflow below 2^31 elements; E - e in
//      [32, 64) goes the same way to window 1; anything smaller (rare for
//      weights: a wave checks each chunk and takes the window-0-only path
//      when it can) adds m to a per-exponent bin in LDS.  All sums are
//      integers, so atomics in any order give the same totals;
//   4. one wave turns the integers into s (a 384-bit sum divided by M*K
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

// float32 bits of 8 consecutive elements.  Non-temporal: each pass streams
// the whole matrix once (a 70B-class matrix is far larger than the caches),
// so its lines should not displace anything (+2-4 % per quantization).
__device__ __forceinline__ void load_bits8(const float *p, uint32_t (&u)[8]) {
    const v4u a = __builtin_nontemporal_load(to_global(reinterpret_cast<const v4u *>(p)));
    const v4u b = __builtin_nontemporal_load(to_global(reinterpret_cast<const v4u *>(p) + 1));
    u[0] = a.x; u[1] = a.y; u[2] = a.z; u[3] = a.w;
    u[4] = b.x; u[5] = b.y; u[6] = b.z; u[7] = b.w;
}
__device__ __forceinline__ void load_bits8(const uint16_t *p, uint32_t (&u)[8]) {
    const v4u a = __builtin_nontemporal_load(to_global(reinterpret_cast<const v4u *>(p)));
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

// Low significand bits that are zero in every element of a T: a bfloat16
// widened to float32 has 16.  Window terms are formed from m >> kZ, so the
// totals carry the unit 2^kZ (the finalize adds it back).
template <typename T> struct ZeroBits;
template <> struct ZeroBits<float> { static constexpr int value = 0; };
template <> struct ZeroBits<uint16_t> { static constexpr int value = 16; };

// Totals of one thread, in the order of WqState::win: window 0 low / high
// 32-bit halves, window 1 low / high halves.  Each window term is below
// 2^(55 - kZ); terms are first summed in 64 bits (at most 2^(8 + kZ) of
// them, so no overflow) and then folded into the halves, which cannot
// overflow below 2^31 elements.
struct WinAcc {
    unsigned long long v[4];
    unsigned long long s0, s1;  // window sums since the last fold
    __host__ __device__ void fold() {
        v[0] += (uint32_t)s0;
        v[1] += s0 >> 32;
        v[2] += (uint32_t)s1;
        v[3] += s1 >> 32;
        s0 = s1 = 0;
    }
};

// Splits |bits| into significand m (hidden bit included) and exponent e
// (at least 1: subnormals share exponent 1), value m * 2^(e - 150).
__host__ __device__ inline void split(uint32_t bits, uint32_t &e, uint32_t &m) {
    const uint32_t a = bits & 0x7FFFFFFFu;
    const uint32_t ef = a >> 23;
    m = (a & 0x7FFFFFu) | (ef != 0u ? 0x800000u : 0u);
    e = ef > 1u ? ef : 1u;
}

// Any element: window 0 or 1, else (returns true) the per-exponent bin.
template <int kZ>
__host__ __device__ inline bool accumulate(uint32_t bits, uint32_t E, WinAcc &acc,
                                           uint32_t &e, uint32_t &m) {
    split(bits, e, m);
    const uint32_t dd = E - e;  // |bits| <= max, so e <= E
    const uint32_t mz = m >> kZ;
    acc.s0 += dd < 32u ? (uint64_t)mz << (31u - dd) : 0ull;
    acc.s1 += dd - 32u < 32u ? (uint64_t)mz << (63u - dd) : 0ull;
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
    constexpr int kZ = ZeroBits<T>::value;
    constexpr int kFold = (1 << (8 + kZ)) / 8;  // chunks of 8 between folds
    __shared__ unsigned long long bins[256];
    __shared__ unsigned long long red[4][kWqWaves];
    for (int i = threadIdx.x; i < 256; i += kWqThreads) bins[i] = 0;
    __syncthreads();
    // exponent field of the max, at least 1
    const uint32_t E = max(__builtin_amdgcn_readfirstlane(st->max_bits) >> 23, 1u);
    WinAcc acc{};
    int since = 0;
    for (int64_t c = (int64_t)blockIdx.x * kWqThreads + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * kWqThreads) {
        uint32_t u[8];
        load_bits8(w + 8 * c, u);
        // Common case, decided per wave: every nonzero element within 32
        // binades of the max, so only window 0 is touched.
        uint32_t far = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t e, m;
            split(u[i], e, m);
            far |= (E - e >= 32u && m != 0u) ? 1u : 0u;
        }
        if (!__any((int)far)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t e, m;
                split(u[i], e, m);
                const uint32_t dd = min(E - e, 31u);  // zeros (m = 0) add 0
                acc.s0 += (uint64_t)(m >> kZ) << (31u - dd);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t e, m;
                if (accumulate<kZ>(u[i], E, acc, e, m))
                    atomicAdd(&bins[e], (unsigned long long)m);
            }
        }
        if (++since == kFold) {
            acc.fold();
            since = 0;
        }
    }
    acc.fold();
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

// 384-bit unsigned integer, 32-bit limbs, least significant first.  Every
// loop is unrolled over the limbs with compares instead of indexing, so the
// limbs stay in registers.
constexpr int kLimbs = 12;

// x += v * 2^shift (0 <= shift, and the sum fits).
__host__ __device__ inline void big_add(uint32_t (&x)[kLimbs], unsigned long long v, int shift) {
    const int j = shift >> 5, r = shift & 31;
    const unsigned long long lo = v << r;
    const uint32_t p0 = (uint32_t)lo, p1 = (uint32_t)(lo >> 32);
    const uint32_t p2 = r ? (uint32_t)(v >> (64 - r)) : 0u;
    unsigned long long carry = 0;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) {
        const uint32_t add = k == j ? p0 : (k == j + 1 ? p1 : (k == j + 2 ? p2 : 0u));
        const unsigned long long t = (unsigned long long)x[k] + add + carry;
        x[k] = (uint32_t)t;
        carry = t >> 32;
    }
}

__host__ __device__ inline uint32_t big_limb(const uint32_t (&x)[kLimbs], int j) {
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) v = k == j ? x[k] : v;
    return v;
}

__host__ __device__ inline int big_bits(const uint32_t (&x)[kLimbs]) {  // bit length
    int b = 0;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) b = x[k] != 0u ? 32 * k + 32 - __builtin_clz(x[k]) : b;
    return b;
}

__host__ __device__ inline bool big_any_below(const uint32_t (&x)[kLimbs], int i) {  // bits [0, i)
    uint32_t any = 0;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) {
        const int n = i - 32 * k;
        const uint32_t mask = n >= 32 ? 0xFFFFFFFFu : (n > 0 ? (1u << n) - 1u : 0u);
        any |= x[k] & mask;
    }
    return any != 0u;
}

// The exact mean, in three steps: X = the windows' totals in units of 2^B
// (mean_begin), plus each bin (mean_add_bin), then X / n rounded once
// (mean_round).  B = min(E - 213, -149) lies at or below every unit used.
struct ExactSum {
    uint32_t x[kLimbs];
    int B;
};

__host__ __device__ inline void mean_begin(ExactSum &S, const WqState *st, int kZ) {
    const int E = st->max_bits >> 23 > 1u ? (int)(st->max_bits >> 23) : 1;
    S.B = E - 213 < -149 ? E - 213 : -149;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) S.x[k] = 0u;
    big_add(S.x, st->win[0], E - 181 + kZ - S.B);       // window 0, low halves
    big_add(S.x, st->win[1], E - 181 + kZ + 32 - S.B);  // window 0, high halves
    big_add(S.x, st->win[2], E - 213 + kZ - S.B);       // window 1, low halves
    big_add(S.x, st->win[3], E - 213 + kZ + 32 - S.B);  // window 1, high halves
}

// Significand sum v of exponent e (e >= 1): v * 2^(e - 150).
__host__ __device__ inline void mean_add_bin(ExactSum &S, int e, unsigned long long v) {
    big_add(S.x, v, e - 150 - S.B);
}

__host__ __device__ inline float mean_round(ExactSum &S, int64_t n) {
    uint32_t (&x)[kLimbs] = S.x;
    const int B = S.B;
    // Q = X / n, R = X % n (n < 2^32, so every step fits 64 bits)
    const unsigned long long nn = (unsigned long long)n;
    unsigned long long rem = 0;
#pragma unroll
    for (int k = kLimbs - 1; k >= 0; --k) {
        const unsigned long long cur = (rem << 32) | x[k];
        x[k] = (uint32_t)(cur / nn);
        rem = cur % nn;
    }
    // keep 24 significant bits, or the bits down to 2^-149
    const int p = big_bits(x) - 1;                        // -1 when Q == 0
    const int q = p + B - 23 > -149 ? p + B - 23 : -149;  // exponent of the last kept bit
    const int k = q - B;                                   // bits of Q dropped (B <= -149 <= q)
    // bits [k, k + 25) of Q through a 64-bit window (k % 32 + 25 <= 56)
    const unsigned long long win =
        (unsigned long long)big_limb(x, k >> 5) | ((unsigned long long)big_limb(x, (k >> 5) + 1) << 32);
    uint32_t m = (uint32_t)(win >> (k & 31)) & 0x1FFFFFFu;
    bool up;
    if (k == 0) {
        up = 2 * rem > nn || (2 * rem == nn && (m & 1u));
    } else {
        const bool half = ((big_limb(x, (k - 1) >> 5) >> ((k - 1) & 31)) & 1u) != 0u;
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

// One wave: lanes load the 256 bins in parallel, the nonzero ones are
// added one at a time (wave-uniform), every lane computing the same result.
__global__ __launch_bounds__(kWave)
void wq_finalize_kernel(WqState *st, int64_t n, int mode, int kZ, float eps, float *stats) {
    const int lane = threadIdx.x;
    float s;
    if (mode == BT_WSCALE_ABSMAX) {
        s = __uint_as_float(st->max_bits);
    } else {
        ExactSum S;
        mean_begin(S, st, kZ);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned long long b = st->bins[4 * lane + i];
            unsigned long long mask = __ballot(b != 0ull);
            while (mask != 0ull) {
                const int l = __ffsll((long long)mask) - 1;
                mask &= mask - 1ull;
                const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
                mean_add_bin(S, 4 * l + i, ((unsigned long long)hi << 32) | lo);
            }
        }
        s = mean_round(S, n);
    }
    const float d = __fadd_rn(s, eps);
    if (lane == 0) {
        st->s = s;
        st->d = d;
        st->thr_bits = code_threshold(d);
        if (stats != nullptr) {
            stats[0] = s;
            stats[1] = d;
        }
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
    hipLaunchKernelGGL(wq_finalize_kernel, dim3(1), dim3(kWave), 0, s, st, n, mode,
                       ZeroBits<T>::value, eps, stats);
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
