// quant.hip -- per-token absmax int8 activation quantization kernel.
//
// The arithmetic (and its page citations) is in quant.hpp, shared with the
// fused prologue of the decode kernel.  The code sum lets the products use
// the codes 0/1/2 directly: sum_k (code - 1) * xq = sum_k code * xq - sum xq.
//
// One workgroup per token; 256 threads sweep the row twice with 16-byte
// loads (the second sweep hits L2).

#include "internal.hpp"
#include "quant.hpp"

namespace bt {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantWaves = kQuantThreads / kWave;

template <typename T>
__global__ __launch_bounds__(kQuantThreads)
void quant_kernel(const T *__restrict__ x, int64_t K, int8_t *__restrict__ xq,
                  float *__restrict__ xs, int32_t *__restrict__ xsum) {
    __shared__ uint32_t red_m[kQuantWaves];
    __shared__ int red_i[kQuantWaves];
    const int64_t n = blockIdx.x;
    const T *row = x + n * K;
    int8_t *out = xq + n * K;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;

    uint32_t mbits = 0;
    for (int64_t k = 8 * (int64_t)threadIdx.x; k < K; k += 8 * kQuantThreads) {
        Raw8<T> r;
        r.load(row + k);
        mbits = max(mbits, r.abs_bits());
    }
    mbits = wave_max_u32(mbits);
    if (lane == 0) red_m[wave] = mbits;
    __syncthreads();
    mbits = red_m[0];
#pragma unroll
    for (int w = 1; w < kQuantWaves; ++w) mbits = max(mbits, red_m[w]);
    const float amax = __uint_as_float(mbits);

    const float inv = quant_inv(amax);
    int sum = 0;
    for (int64_t k = 8 * (int64_t)threadIdx.x; k < K; k += 8 * kQuantThreads) {
        Raw8<T> r;
        r.load(row + k);
        *reinterpret_cast<uint2 *>(out + k) = quant8(r.eight(), inv, sum);
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
