// quant.hip -- per-token absmax int8 activation quantization kernel.
//
// The arithmetic (and its page citations) is in quant.hpp, shared with the
// fused prologues of the decode kernels.  The code sum lets the products use
// the codes 0/1/2 directly: sum_k (code - 1) * xq = sum_k code * xq - sum xq.
//
// One workgroup per token and input (several inputs of the same tokens can
// share one launch), of 128, 256 or 512 threads: the fewest that keep the
// longest row within 8 chunks per thread (small workgroups turn over faster
// when there are thousands of rows), but 512 when there are no more rows
// than compute units (each row then has a unit to itself, and eight waves
// spread its rounding over all four SIMDs: 64 tokens of a 2560/6912 block
// 22.3 -> 21.7 us per block with the product; 1024 threads 22.1).  Rows of
// up to 8 * threads * C elements are done in one pass: every thread loads
// all of its C chunks of 8 elements at once
// (no load waits on another), the absmax is reduced in registers, across the
// wave with DPP moves and across the waves through LDS, and the codes are
// rounded from the registers.  Longer rows sweep the row twice (the second
// sweep hits L2).

#include "internal.hpp"
#include "quant.hpp"

namespace bt {

namespace {

constexpr int kQuantThreads = 512;  // two-pass kernel, and the one-pass maximum
constexpr int kQuantWaves = kQuantThreads / kWave;

// Max over the waves' partial maxima / sums written to LDS (after a barrier).
template <bool MAX, int W>
__device__ __forceinline__ uint32_t across_waves(const uint32_t (&part)[W]) {
    uint32_t v = part[0];
#pragma unroll
    for (int w = 1; w < W; ++w) v = MAX ? max(v, part[w]) : v + part[w];
    return v;
}

// One-pass quantization of token blockIdx.x of input blockIdx.y, TH threads.
template <typename T, int C, int TH>
__global__ __launch_bounds__(TH)
void quant_onepass_kernel(QuantJobs jobs) {
    constexpr int kWaves = TH / kWave;
    __shared__ uint32_t red_m[kWaves];
    __shared__ uint32_t red_s[kWaves];
    const int64_t n = blockIdx.x;
    const int job = __builtin_amdgcn_readfirstlane(blockIdx.y);
    const T *x = static_cast<const T *>(jobs.x[0]);
    int8_t *xq = jobs.xq[0];
    float *xs = jobs.xs[0];
    int32_t *xsum = jobs.xsum[0];
    int64_t K = jobs.K[0];
#pragma unroll
    for (int i = 1; i < kMaxQuantJobs; ++i) {
        if (job == i) {
            x = static_cast<const T *>(jobs.x[i]);
            xq = jobs.xq[i];
            xs = jobs.xs[i];
            xsum = jobs.xsum[i];
            K = jobs.K[i];
        }
    }
    const T *row = x + n * K;
    int8_t *out = xq + n * K;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;

    // chunk c of this thread starts at element 8 * (threadIdx.x + c * threads);
    // chunks past the row re-read the last one and are masked
    Raw8<T> raw[C];
#pragma unroll
    for (int c = 0; c < C; ++c)
        raw[c].load(row + min(8 * ((int64_t)threadIdx.x + (int64_t)c * TH), K - 8));
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < C; ++c)  // re-read chunks cannot change a max
        m = max(m, raw[c].abs_bits());
    m = wave_reduce<true>(m);
    if (lane == 0) red_m[wave] = m;
    __syncthreads();
    const float amax = __uint_as_float(across_waves<true>(red_m));
    const float inv = quant_inv(amax);
    int sum = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t k = 8 * ((int64_t)threadIdx.x + (int64_t)c * TH);
        int part = 0;
        const uint2 q = quant8(raw[c].eight(), inv, part);
        if (k < K) {
            *reinterpret_cast<uint2 *>(out + k) = q;
            sum += part;
        }
    }
    const uint32_t s = wave_reduce<false>((uint32_t)sum);
    if (lane == 0) red_s[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        xs[n] = amax;
        xsum[n] = (int32_t)across_waves<false>(red_s);
    }
}

// Rows longer than 8 * threads * (largest C): two sweeps.
template <typename T>
__global__ __launch_bounds__(kQuantThreads)
void quant_twopass_kernel(const T *__restrict__ x, int64_t K, int8_t *__restrict__ xq,
                          float *__restrict__ xs, int32_t *__restrict__ xsum) {
    __shared__ uint32_t red_m[kQuantWaves];
    __shared__ uint32_t red_s[kQuantWaves];
    const int64_t n = blockIdx.x;
    const T *row = x + n * K;
    int8_t *out = xq + n * K;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;

    uint32_t m = 0;
    for (int64_t k = 8 * (int64_t)threadIdx.x; k < K; k += 8 * kQuantThreads) {
        Raw8<T> r;
        r.load(row + k);
        m = max(m, r.abs_bits());
    }
    m = wave_reduce<true>(m);
    if (lane == 0) red_m[wave] = m;
    __syncthreads();
    const float amax = __uint_as_float(across_waves<true>(red_m));
    const float inv = quant_inv(amax);
    int sum = 0;
    for (int64_t k = 8 * (int64_t)threadIdx.x; k < K; k += 8 * kQuantThreads) {
        Raw8<T> r;
        r.load(row + k);
        *reinterpret_cast<uint2 *>(out + k) = quant8(r.eight(), inv, sum);
    }
    const uint32_t s = wave_reduce<false>((uint32_t)sum);
    if (lane == 0) red_s[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        xs[n] = amax;
        xsum[n] = (int32_t)across_waves<false>(red_s);
    }
}

// All jobs in one launch when every row fits the one-pass kernel (the chunk
// count is that of the longest row; shorter rows mask the extra chunks),
// else one two-pass launch per job.
template <typename T, int TH>
void launch_onepass(const QuantJobs &jobs, int64_t chunks, dim3 grid, hipStream_t s) {
    const dim3 block(TH);
    if (chunks <= 1) hipLaunchKernelGGL((quant_onepass_kernel<T, 1, TH>), grid, block, 0, s, jobs);
    else if (chunks <= 2) hipLaunchKernelGGL((quant_onepass_kernel<T, 2, TH>), grid, block, 0, s, jobs);
    else if (chunks <= 4) hipLaunchKernelGGL((quant_onepass_kernel<T, 4, TH>), grid, block, 0, s, jobs);
    else hipLaunchKernelGGL((quant_onepass_kernel<T, 8, TH>), grid, block, 0, s, jobs);
}

template <typename T>
hipError_t launch_quant_t(const QuantJobs &jobs, int count, int64_t N, hipStream_t s) {
    int64_t kmax = 0;
    for (int i = 0; i < count; ++i) kmax = max(kmax, jobs.K[i]);
    const int64_t units = kmax / 8;  // 8-element chunks of the longest row
    const dim3 grid((unsigned)N, (unsigned)count);
    if (N * count <= device_cus() && units <= 512 * 8)
        launch_onepass<T, 512>(jobs, (units + 511) / 512, grid, s);
    else if (units <= 128 * 8) launch_onepass<T, 128>(jobs, (units + 127) / 128, grid, s);
    else if (units <= 256 * 8) launch_onepass<T, 256>(jobs, (units + 255) / 256, grid, s);
    else if (units <= 512 * 8) launch_onepass<T, 512>(jobs, (units + 511) / 512, grid, s);
    else
        for (int i = 0; i < count; ++i)
            hipLaunchKernelGGL(quant_twopass_kernel<T>, dim3((unsigned)N), dim3(kQuantThreads), 0, s,
                               static_cast<const T *>(jobs.x[i]), jobs.K[i], jobs.xq[i], jobs.xs[i],
                               jobs.xsum[i]);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_jobs(const QuantJobs &jobs, int count, bt_dtype xdt, int64_t N,
                             hipStream_t s) {
    if (N == 0 || count == 0) return hipSuccess;
    QuantJobs j = jobs;
    for (int i = count; i < kMaxQuantJobs; ++i) {  // unused entries repeat the first
        j.x[i] = j.x[0];
        j.K[i] = j.K[0];
        j.xq[i] = j.xq[0];
        j.xs[i] = j.xs[0];
        j.xsum[i] = j.xsum[0];
    }
    if (xdt == BT_F32) return launch_quant_t<float>(j, count, N, s);
    return launch_quant_t<uint16_t>(j, count, N, s);
}

hipError_t launch_quant(const void *x, bt_dtype xdt, int64_t N, int64_t K,
                        int8_t *xq, float *xs, int32_t *xsum, hipStream_t s) {
    QuantJobs j{};
    j.x[0] = x;
    j.K[0] = K;
    j.xq[0] = xq;
    j.xs[0] = xs;
    j.xsum[0] = xsum;
    return launch_quant_jobs(j, 1, xdt, N, s);
}

}  // namespace bt
