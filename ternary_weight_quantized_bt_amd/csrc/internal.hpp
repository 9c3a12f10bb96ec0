// internal.hpp -- host-side launchers behind the C ABI (validated arguments
// only; every function enqueues on `s` and returns hipGetLastError()).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libternary.h"

namespace bt {

hipError_t launch_pack(const int8_t *w, int64_t M, int64_t K, float scale,
                       uint8_t *packed, int32_t *invalid, hipStream_t s);
hipError_t launch_unpack(const uint8_t *packed, int64_t M, int64_t K,
                         int8_t *w, hipStream_t s);
hipError_t launch_dequant(const uint8_t *packed, int64_t M, int64_t K, void *w, bt_dtype wdt,
                          hipStream_t s);
hipError_t launch_i2s_import(const uint8_t *src, int64_t M, int64_t K, int64_t block,
                             uint8_t *packed, int32_t *invalid, hipStream_t s);
hipError_t launch_i2s_export(const uint8_t *packed, int64_t M, int64_t K, int64_t block,
                             uint8_t *dst, hipStream_t s);
// Base-3 "B3T1024" weights: packing, unpacking, decode product (any N).
hipError_t launch_b3_pack(const int8_t *w, int64_t M, int64_t K, float scale, uint8_t *packed,
                          int32_t *invalid, hipStream_t s);
hipError_t launch_b3_unpack(const uint8_t *packed, int64_t M, int64_t K, int8_t *w,
                            hipStream_t s);
hipError_t launch_b3_gemv(const uint8_t *packed, int64_t M, int64_t K, const int8_t *xq,
                          const float *xs, const int32_t *xsum, int64_t N, void *y,
                          bt_dtype ydt, hipStream_t s);
// Float -> packed ternary weights (workspace: BT_WQ_WORKSPACE_BYTES).
hipError_t launch_quantize_weights(const void *w, bt_dtype wdt, int64_t M, int64_t K, int mode,
                                   float eps, uint8_t *packed, float *stats, void *workspace,
                                   hipStream_t s);
hipError_t launch_quant(const void *x, bt_dtype xdt, int64_t N, int64_t K,
                        int8_t *xq, float *xs, int32_t *xsum, hipStream_t s);
// Several inputs of N tokens each (widths K[i]) quantized in one launch.
constexpr int kMaxQuantJobs = 4;
struct QuantJobs {
    const void *x[kMaxQuantJobs];
    int64_t K[kMaxQuantJobs];
    int8_t *xq[kMaxQuantJobs];
    float *xs[kMaxQuantJobs];
    int32_t *xsum[kMaxQuantJobs];
};
hipError_t launch_quant_jobs(const QuantJobs &jobs, int count, bt_dtype xdt, int64_t N,
                             hipStream_t s);

// One projection of a grouped launch.
struct Proj {
    const uint8_t *packed;
    int64_t M;
    void *y;
};
constexpr int kMaxGroup = 3;
struct Group {
    Proj p[kMaxGroup];
    int count;
    int64_t K;                 // shared by every projection of the group
    const int8_t *xq;          // [N, K]
    const float *xs;           // [N]
    const int32_t *xsum;       // [N]
    int64_t N;
    bt_dtype ydt;
};

// Decode path (few tokens): 128-bit weight streaming + dot4, or skinny
// matrix-core tiles where those are faster (decode_dot4).
hipError_t launch_decode(const Group &g, hipStream_t s);
// Whether the decode of N tokens over a group of M rows (all its
// projections) and K columns runs on the dot4 kernel (else the matrix cores).
bool decode_dot4(int64_t N, int64_t M, int64_t K);
// Rows of a group (all its projections).
inline int64_t group_rows(const Group &g) {
    int64_t m = 0;
    for (int j = 0; j < g.count; ++j) m += g.p[j].M;
    return m;
}
// Decode path with the activation quantization fused into the kernel's
// prologue (x is the float / bf16 input of the group).  Only for shapes where
// decode_fuses_quant(N, M, K) holds.
bool decode_fuses_quant(int64_t N, int64_t M, int64_t K, bt_dtype xdt);
// Matrix-core decode (1 < N < BT_PREFILL_MIN_N) of up to four groups,
// each with its own quantized input, in one launch; results equal
// launch_decode per group.
hipError_t launch_decode_groups(const Group *groups, int count, hipStream_t s);
hipError_t launch_decode_fused(const Group &g, const void *x, bt_dtype xdt, hipStream_t s);
// Prefill path: tiled int8 matrix-core product.
hipError_t launch_prefill(const Group &g, hipStream_t s);
// Prefill of up to four groups, each with its own quantized input, in one
// launch; results equal launch_prefill per group.
hipError_t launch_prefill_groups(const Group *groups, int count, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cus();

// Largest N for which launch_decode may use the dot4 kernel.
constexpr int64_t kDot4MaxN = 4;
// Largest N launch_decode takes: the matrix-core decode lays its 16-token
// groups along the grid's y axis, at most 65535 of them.
constexpr int64_t kDecodeMaxN = 65535 * 16;

// The per-layer driver behind bt_layer_forward with its scratch passed
// explicitly (`fn` names the entry point in error messages), and its argument
// checks alone: every check but the workspace's, and the scratch bytes the
// call needs (0 when it launches nothing).  Host only; no GPU call.
bt_status layer_forward(const bt_layer *L, const bt_layer_io *io, void *workspace,
                        size_t workspace_bytes, bt_stream stream, const char *fn);
bt_status layer_check(const bt_layer *L, const bt_layer_io *io, const char *fn,
                      size_t *scratch_bytes);
// Records `msg` as the calling thread's last error and returns st.
bt_status fail_with(bt_status st, const char *msg);

}  // namespace bt
