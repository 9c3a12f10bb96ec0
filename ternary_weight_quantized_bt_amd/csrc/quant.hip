// quant.hip -- per-token absmax int8 activation quantization.
//
// [PARA] section 5 ("The Mathematics of BitNet b1.58"): activations are
// quantized to 8-bit integers with one AbsMax scale per token (Quant8).  The
// pages print no formula; the one implemented (and stated in libternary.h):
//   amax = max|x| (float32, exact for any order), inv = 127 / amax (float32,
//   correctly rounded), xq = clamp(rne(x * inv), -127, 127) (float32
//   multiply, round half to even), scale = amax, sum = sum of xq.
// The sum lets the product use the codes 0/1/2 directly:
//   sum_k (code - 1) * xq = sum_k code * xq - sum_k xq.
//
// One workgroup per token; 256 threads sweep the row twice with 16-byte
// loads (the second sweep hits L2).  Explicit __fdiv_rn / __fmul_rn keep the
// division correctly rounded and the product unfused whatever the compiler
// flags; rintf is round-half-to-even.

#include "common.hpp"
#include "internal.hpp"

namespace bt {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;

// Eight consecutive inputs widened to float32.
struct Eight {
    float v[8];
};

__device__ __forceinline__ Eight load8(const float *p) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    return Eight{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
}

__device__ __forceinline__ Eight load8(const uint16_t *p) {
    const uint4 a = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    Eight e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e.v[2 * i] = __uint_as_float(w[i] << 16);
        e.v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    return e;
}

__device__ __forceinline__ int quant1(float x, float inv) {
    float r = rintf(__fmul_rn(x, inv));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

template <typename T>
__global__ __launch_bounds__(kQuantThreads)
void quant_kernel(const T *__restrict__ x, int64_t K, int8_t *__restrict__ xq,
                  float *__restrict__ xs, int32_t *__restrict__ xsum) {
    __shared__ float red_f[kQuantWaves];
    __shared__ int red_i[kQuantWaves];
    const int64_t n = blockIdx.x;
    const T *row = x + n * K;
    int8_t *out = xq + n * K;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;

    float amax = 0.0f;
    for (int64_t k = 8 * (int64_t)threadIdx.x; k < K; k += 8 * kQuantThreads) {
        const Eight e = load8(row + k);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(e.v[i]));
    }
    amax = wave_max(amax);
    if (lane == 0) red_f[wave] = amax;
    __syncthreads();
    amax = red_f[0];
#pragma unroll
    for (int w = 1; w < kQuantWaves; ++w) amax = fmaxf(amax, red_f[w]);

    int sum = 0;
    if (amax == 0.0f) {
        for (int64_t k = 8 * (int64_t)threadIdx.x; k < K; k += 8 * kQuantThreads)
            *reinterpret_cast<uint2 *>(out + k) = make_uint2(0u, 0u);
    } else {
        const float inv = __fdiv_rn(127.0f, amax);
        for (int64_t k = 8 * (int64_t)threadIdx.x; k < K; k += 8 * kQuantThreads) {
            const Eight e = load8(row + k);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int a = quant1(e.v[i], inv);
                const int b = quant1(e.v[4 + i], inv);
                sum += a + b;
                lo |= ((uint32_t)a & 0xFFu) << (8 * i);
                hi |= ((uint32_t)b & 0xFFu) << (8 * i);
            }
            *reinterpret_cast<uint2 *>(out + k) = make_uint2(lo, hi);
        }
    }
    sum = wave_sum(sum);
    if (lane == 0) red_i[wave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        int total = 0;
#pragma unroll
        for (int w = 0; w < kQuantWaves; ++w) total += red_i[w];
        xs[n] = amax;
        xsum[n] = total;
    }
}

}  // namespace

hipError_t launch_quant(const void *x, bt_dtype xdt, int64_t N, int64_t K,
                        int8_t *xq, float *xs, int32_t *xsum, hipStream_t s) {
    if (N == 0) return hipSuccess;
    if (xdt == BT_F32)
        hipLaunchKernelGGL(quant_kernel<float>, dim3((unsigned)N),
                           dim3(kQuantThreads), 0, s,
                           static_cast<const float *>(x), K, xq, xs, xsum);
    else
        hipLaunchKernelGGL(quant_kernel<uint16_t>, dim3((unsigned)N),
                           dim3(kQuantThreads), 0, s,
                           static_cast<const uint16_t *>(x), K, xq, xs, xsum);
    return hipGetLastError();
}

}  // namespace bt
