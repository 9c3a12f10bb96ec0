// api.hip -- the C ABI of libternary: argument validation, dispatch, and the
// per-layer projection driver.  Host code only; kernels live in the other
// files.  Nothing here allocates, frees or synchronizes.
//
// The seven projections of a block ("BitNet Inference Preprocessing:
// Converting Hugging Face Checkpoints to I2S GGUF", "Stage 1": q, k, v, o,
// gate, up, down) are run as four groups that share one quantized input.

#include <stdarg.h>
#include <stdio.h>

#include "internal.hpp"
#include "layer.hpp"

namespace {

thread_local char g_err[512] = "";

bt_status fail(bt_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bt_status ok() {
    g_err[0] = '\0';
    return BT_OK;
}

bt_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess)
        return fail(BT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bt_status check_mk(int64_t M, int64_t K, const char *fn) {
    if (M <= 0 || K <= 0)
        return fail(BT_ERR_SHAPE, "%s: M and K must be positive (M=%lld, K=%lld)", fn,
                    (long long)M, (long long)K);
    if (M % 16 != 0)
        return fail(BT_ERR_SHAPE, "%s: M=%lld is not a multiple of 16", fn, (long long)M);
    if (K % 256 != 0)
        return fail(BT_ERR_SHAPE, "%s: K=%lld is not a multiple of 256", fn, (long long)K);
    if (K > BT_MAX_K)
        return fail(BT_ERR_SHAPE, "%s: K=%lld exceeds %d", fn, (long long)K, BT_MAX_K);
    if (M > (int64_t)1 << 40)
        return fail(BT_ERR_SHAPE, "%s: M=%lld too large", fn, (long long)M);
    return BT_OK;
}

bt_status check_ptr(const void *p, const char *name, const char *fn) {
    if (p == nullptr) return fail(BT_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
    if (!aligned16(p)) return fail(BT_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, name);
    return BT_OK;
}

bt_status check_n(int64_t N, const char *fn) {
    if (N < 0) return fail(BT_ERR_INVALID_ARG, "%s: N=%lld is negative", fn, (long long)N);
    if (N > BT_MAX_N)
        return fail(BT_ERR_SHAPE, "%s: N=%lld exceeds %d", fn, (long long)N, BT_MAX_N);
    return BT_OK;
}

#define BT_TRY(expr)                        \
    do {                                    \
        const bt_status st_ = (expr);       \
        if (st_ != BT_OK) return st_;       \
    } while (0)

hipStream_t as_stream(bt_stream s) { return reinterpret_cast<hipStream_t>(s); }

bt_status check_matmul(const char *fn, const uint8_t *packed, int64_t M, int64_t K,
                       const int8_t *xq, const float *xs, const int32_t *xsum,
                       int64_t N, void *y, bt_dtype ydt) {
    BT_TRY(check_mk(M, K, fn));
    BT_TRY(check_n(N, fn));
    if (ydt != BT_F32 && ydt != BT_BF16 && ydt != BT_I32)
        return fail(BT_ERR_DTYPE, "%s: unsupported y dtype %d", fn, (int)ydt);
    BT_TRY(check_ptr(packed, "packed", fn));
    if (N == 0) return BT_OK;
    BT_TRY(check_ptr(xq, "xq", fn));
    if (xs == nullptr) return fail(BT_ERR_INVALID_ARG, "%s: x_scale is NULL", fn);
    if (xsum == nullptr) return fail(BT_ERR_INVALID_ARG, "%s: x_sum is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(xs) & 3u) || (reinterpret_cast<uintptr_t>(xsum) & 3u))
        return fail(BT_ERR_ALIGN, "%s: x_scale / x_sum not 4-byte aligned", fn);
    BT_TRY(check_ptr(y, "y", fn));
    return BT_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace carve-up for a layer: per input i, xq_i [N, K_i], then scales and
// sums [N] each, every block 256-byte aligned.
struct LayerWs {
    int8_t *xq[BT_LAYER_INPUTS];
    float *xs[BT_LAYER_INPUTS];
    int32_t *xsum[BT_LAYER_INPUTS];
    size_t bytes;
};

bool layer_input_widths(const bt_layer *L, int64_t Kin[BT_LAYER_INPUTS]) {
    if (L->K[0] != L->K[1] || L->K[0] != L->K[2] || L->K[4] != L->K[5]) return false;
    Kin[0] = L->K[0];
    Kin[1] = L->K[3];
    Kin[2] = L->K[4];
    Kin[3] = L->K[6];
    return true;
}

LayerWs carve(const int64_t Kin[BT_LAYER_INPUTS], int64_t N, void *base) {
    LayerWs w{};
    size_t off = 0;
    uint8_t *b = static_cast<uint8_t *>(base);
    for (int i = 0; i < BT_LAYER_INPUTS; ++i) {
        w.xq[i] = reinterpret_cast<int8_t *>(b + off);
        off = align256(off + (size_t)N * (size_t)Kin[i]);
        w.xs[i] = reinterpret_cast<float *>(b + off);
        off = align256(off + (size_t)N * sizeof(float));
        w.xsum[i] = reinterpret_cast<int32_t *>(b + off);
        off = align256(off + (size_t)N * sizeof(int32_t));
    }
    w.bytes = off;
    return w;
}

static_assert(BT_MAX_GROUP == bt::kMaxGroup, "group size");

hipError_t run_group(const bt::Group &g, hipStream_t s) {
    return g.N >= BT_PREFILL_MIN_N ? bt::launch_prefill(g, s) : bt::launch_decode(g, s);
}

}  // namespace

extern "C" {

int bt_abi_version(void) { return BT_ABI_VERSION; }

const char *bt_last_error(void) { return g_err; }

size_t bt_packed_bytes(int64_t M, int64_t K) {
    if (check_mk(M, K, "bt_packed_bytes") != BT_OK) return 0;
    ok();
    return (size_t)(M * K / 4) + BT_TAIL_BYTES;
}

bt_status bt_pack_ternary(const int8_t *w, int64_t M, int64_t K, float scale,
                          uint8_t *packed, int32_t *invalid_count, bt_stream stream) {
    const char *fn = "bt_pack_ternary";
    BT_TRY(check_mk(M, K, fn));
    BT_TRY(check_ptr(w, "w", fn));
    BT_TRY(check_ptr(packed, "packed", fn));
    if (invalid_count && (reinterpret_cast<uintptr_t>(invalid_count) & 3u))
        return fail(BT_ERR_ALIGN, "%s: invalid_count not 4-byte aligned", fn);
    return hip_status(bt::launch_pack(w, M, K, scale, packed, invalid_count, as_stream(stream)), fn);
}

bt_status bt_unpack_ternary(const uint8_t *packed, int64_t M, int64_t K, int8_t *w,
                            bt_stream stream) {
    const char *fn = "bt_unpack_ternary";
    BT_TRY(check_mk(M, K, fn));
    BT_TRY(check_ptr(packed, "packed", fn));
    BT_TRY(check_ptr(w, "w", fn));
    return hip_status(bt::launch_unpack(packed, M, K, w, as_stream(stream)), fn);
}

size_t bt_i2s_bytes(int64_t M, int64_t K) {
    if (check_mk(M, K, "bt_i2s_bytes") != BT_OK) return 0;
    return (size_t)(M * K / 4) + 4;
}

bt_status bt_dequantize_weights(const uint8_t *packed, int64_t M, int64_t K, void *w,
                                bt_dtype w_dtype, bt_stream stream) {
    const char *fn = "bt_dequantize_weights";
    BT_TRY(check_mk(M, K, fn));
    if (w_dtype != BT_F32 && w_dtype != BT_BF16)
        return fail(BT_ERR_DTYPE, "%s: w dtype must be BT_F32 or BT_BF16", fn);
    BT_TRY(check_ptr(packed, "packed", fn));
    BT_TRY(check_ptr(w, "w", fn));
    return hip_status(bt::launch_dequant(packed, M, K, w, w_dtype, as_stream(stream)), fn);
}

static bt_status check_i2s_block(int64_t M, int64_t K, int64_t block, const char *fn) {
    if (block <= 0 || block % 4 != 0 || block > ((int64_t)1 << 31) || (M * K) % block != 0)
        return fail(BT_ERR_SHAPE, "%s: block=%lld must be a positive multiple of 4 dividing M*K",
                    fn, (long long)block);
    return BT_OK;
}

bt_status bt_i2s_import(const uint8_t *i2s, int64_t M, int64_t K, int64_t block,
                        uint8_t *packed, int32_t *invalid_count, bt_stream stream) {
    const char *fn = "bt_i2s_import";
    BT_TRY(check_mk(M, K, fn));
    BT_TRY(check_i2s_block(M, K, block, fn));
    BT_TRY(check_ptr(i2s, "i2s", fn));
    BT_TRY(check_ptr(packed, "packed", fn));
    if (invalid_count != nullptr && (reinterpret_cast<uintptr_t>(invalid_count) & 3u))
        return fail(BT_ERR_ALIGN, "%s: invalid_count is not 4-byte aligned", fn);
    return hip_status(
        bt::launch_i2s_import(i2s, M, K, block, packed, invalid_count, as_stream(stream)), fn);
}

bt_status bt_i2s_export(const uint8_t *packed, int64_t M, int64_t K, int64_t block,
                        uint8_t *i2s, bt_stream stream) {
    const char *fn = "bt_i2s_export";
    BT_TRY(check_mk(M, K, fn));
    BT_TRY(check_i2s_block(M, K, block, fn));
    BT_TRY(check_ptr(packed, "packed", fn));
    BT_TRY(check_ptr(i2s, "i2s", fn));
    return hip_status(bt::launch_i2s_export(packed, M, K, block, i2s, as_stream(stream)), fn);
}

static bt_status check_b3(int64_t M, int64_t K, const char *fn) {
    BT_TRY(check_mk(M, K, fn));
    if (K % 1024 != 0)
        return fail(BT_ERR_SHAPE, "%s: K=%lld is not a multiple of 1024", fn, (long long)K);
    return BT_OK;
}

size_t bt_b3_bytes(int64_t M, int64_t K) {
    if (check_b3(M, K, "bt_b3_bytes") != BT_OK) return 0;
    ok();
    return (size_t)(M * K / 64 * 13) + BT_TAIL_BYTES;
}

bt_status bt_pack_ternary_b3(const int8_t *w, int64_t M, int64_t K, float scale,
                             uint8_t *packed, int32_t *invalid_count, bt_stream stream) {
    const char *fn = "bt_pack_ternary_b3";
    BT_TRY(check_b3(M, K, fn));
    BT_TRY(check_ptr(w, "w", fn));
    BT_TRY(check_ptr(packed, "packed", fn));
    if (invalid_count && (reinterpret_cast<uintptr_t>(invalid_count) & 3u))
        return fail(BT_ERR_ALIGN, "%s: invalid_count not 4-byte aligned", fn);
    return hip_status(bt::launch_b3_pack(w, M, K, scale, packed, invalid_count,
                                         as_stream(stream)), fn);
}

bt_status bt_unpack_ternary_b3(const uint8_t *packed, int64_t M, int64_t K, int8_t *w,
                               bt_stream stream) {
    const char *fn = "bt_unpack_ternary_b3";
    BT_TRY(check_b3(M, K, fn));
    BT_TRY(check_ptr(packed, "packed", fn));
    BT_TRY(check_ptr(w, "w", fn));
    return hip_status(bt::launch_b3_unpack(packed, M, K, w, as_stream(stream)), fn);
}

bt_status bt_ternary_gemv_b3(const uint8_t *packed, int64_t M, int64_t K, const int8_t *xq,
                             const float *x_scale, const int32_t *x_sum, int64_t N, void *y,
                             bt_dtype y_dtype, bt_stream stream) {
    const char *fn = "bt_ternary_gemv_b3";
    BT_TRY(check_b3(M, K, fn));
    BT_TRY(check_matmul(fn, packed, M, K, xq, x_scale, x_sum, N, y, y_dtype));
    if (N == 0) return ok();
    return hip_status(bt::launch_b3_gemv(packed, M, K, xq, x_scale, x_sum, N, y, y_dtype,
                                         as_stream(stream)), fn);
}

size_t bt_quantize_weights_workspace_bytes(void) { return BT_WQ_WORKSPACE_BYTES; }

bt_status bt_quantize_weights(const void *w, bt_dtype w_dtype, int64_t M, int64_t K,
                              int scale_mode, float eps, uint8_t *packed, float *stats,
                              void *workspace, size_t workspace_bytes, bt_stream stream) {
    const char *fn = "bt_quantize_weights";
    BT_TRY(check_mk(M, K, fn));
    if (M > ((int64_t)1 << 31) / K)
        return fail(BT_ERR_SHAPE, "%s: M*K=%lld exceeds 2^31", fn, (long long)(M * K));
    if (w_dtype != BT_F32 && w_dtype != BT_BF16)
        return fail(BT_ERR_DTYPE, "%s: w dtype must be BT_F32 or BT_BF16", fn);
    if (scale_mode != BT_WSCALE_ABSMEAN && scale_mode != BT_WSCALE_ABSMAX)
        return fail(BT_ERR_INVALID_ARG, "%s: unknown scale mode %d", fn, scale_mode);
    if (!(eps >= 0.0f && eps <= 3.402823466e38f))
        return fail(BT_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
    BT_TRY(check_ptr(w, "w", fn));
    BT_TRY(check_ptr(packed, "packed", fn));
    if (stats != nullptr && (reinterpret_cast<uintptr_t>(stats) & 3u))
        return fail(BT_ERR_ALIGN, "%s: stats is not 4-byte aligned", fn);
    if (workspace == nullptr || workspace_bytes < BT_WQ_WORKSPACE_BYTES)
        return fail(BT_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn,
                    (size_t)BT_WQ_WORKSPACE_BYTES);
    BT_TRY(check_ptr(workspace, "workspace", fn));
    return hip_status(bt::launch_quantize_weights(w, w_dtype, M, K, scale_mode, eps, packed,
                                                  stats, workspace, as_stream(stream)),
                      fn);
}

bt_status bt_quant_act(const void *x, bt_dtype x_dtype, int64_t N, int64_t K, int8_t *xq,
                       float *x_scale, int32_t *x_sum, bt_stream stream) {
    const char *fn = "bt_quant_act";
    BT_TRY(check_n(N, fn));
    if (x_dtype != BT_F32 && x_dtype != BT_BF16)
        return fail(BT_ERR_DTYPE, "%s: x dtype must be BT_F32 or BT_BF16", fn);
    if (K <= 0 || K % 256 != 0 || K > BT_MAX_K)
        return fail(BT_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 256 <= %d", fn,
                    (long long)K, BT_MAX_K);
    if (N == 0) return ok();
    BT_TRY(check_ptr(x, "x", fn));
    BT_TRY(check_ptr(xq, "xq", fn));
    if (x_scale == nullptr || x_sum == nullptr)
        return fail(BT_ERR_INVALID_ARG, "%s: x_scale / x_sum is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(x_scale) & 3u) || (reinterpret_cast<uintptr_t>(x_sum) & 3u))
        return fail(BT_ERR_ALIGN, "%s: x_scale / x_sum not 4-byte aligned", fn);
    return hip_status(bt::launch_quant(x, x_dtype, N, K, xq, x_scale, x_sum, as_stream(stream)),
                      fn);
}

static bt::Group single_group(const uint8_t *packed, int64_t M, int64_t K, const int8_t *xq,
                              const float *xs, const int32_t *xsum, int64_t N, void *y,
                              bt_dtype ydt) {
    bt::Group g{};
    g.p[0] = bt::Proj{packed, M, y};
    g.count = 1;
    g.K = K;
    g.xq = xq;
    g.xs = xs;
    g.xsum = xsum;
    g.N = N;
    g.ydt = ydt;
    return g;
}

bt_status bt_ternary_gemv(const uint8_t *packed, int64_t M, int64_t K, const int8_t *xq,
                          const float *x_scale, const int32_t *x_sum, int64_t N, void *y,
                          bt_dtype y_dtype, bt_stream stream) {
    const char *fn = "bt_ternary_gemv";
    BT_TRY(check_matmul(fn, packed, M, K, xq, x_scale, x_sum, N, y, y_dtype));
    if (N == 0) return ok();
    const bt::Group g = single_group(packed, M, K, xq, x_scale, x_sum, N, y, y_dtype);
    // more tokens than the decode grid holds: the prefill kernel (same bits)
    return hip_status(N > bt::kDecodeMaxN ? bt::launch_prefill(g, as_stream(stream))
                                          : bt::launch_decode(g, as_stream(stream)),
                      fn);
}

bt_status bt_ternary_gemm(const uint8_t *packed, int64_t M, int64_t K, const int8_t *xq,
                          const float *x_scale, const int32_t *x_sum, int64_t N, void *y,
                          bt_dtype y_dtype, bt_stream stream) {
    const char *fn = "bt_ternary_gemm";
    BT_TRY(check_matmul(fn, packed, M, K, xq, x_scale, x_sum, N, y, y_dtype));
    if (N == 0) return ok();
    const bt::Group g = single_group(packed, M, K, xq, x_scale, x_sum, N, y, y_dtype);
    return hip_status(bt::launch_prefill(g, as_stream(stream)), fn);
}

// Workspace of the two-launch linear path: codes [N, K], scales [N], sums [N],
// each block 256-byte aligned.
static size_t linear_ws_bytes(int64_t N, int64_t K) {
    return align256((size_t)N * (size_t)K) + 2 * align256((size_t)N * sizeof(float));
}

static bool linear_fuses(int64_t N, int64_t M, int64_t K, bt_dtype xdt) {
    return N < BT_PREFILL_MIN_N && bt::decode_fuses_quant(N, M, K, xdt);
}

size_t bt_linear_workspace_bytes(int64_t N, int64_t K) {
    if (N < 0 || N > BT_MAX_N || K <= 0 || K % 256 != 0 || K > BT_MAX_K) return 0;
    return linear_ws_bytes(N, K);
}

int bt_linear_one_launch(int64_t N, int64_t M, int64_t K, bt_dtype x_dtype) {
    if (N < 0 || N > BT_MAX_N || (x_dtype != BT_F32 && x_dtype != BT_BF16)) return -1;
    if (check_mk(M, K, "bt_linear_one_launch") != BT_OK) return -1;
    return N > 0 && linear_fuses(N, M, K, x_dtype) ? 1 : 0;
}

bt_status bt_ternary_linear(const uint8_t *packed, int64_t M, int64_t K, const void *x,
                            bt_dtype x_dtype, int64_t N, void *y, bt_dtype y_dtype,
                            void *workspace, size_t workspace_bytes, bt_stream stream) {
    const char *fn = "bt_ternary_linear";
    BT_TRY(check_mk(M, K, fn));
    BT_TRY(check_n(N, fn));
    if (x_dtype != BT_F32 && x_dtype != BT_BF16)
        return fail(BT_ERR_DTYPE, "%s: x dtype must be BT_F32 or BT_BF16", fn);
    if (y_dtype != BT_F32 && y_dtype != BT_BF16 && y_dtype != BT_I32)
        return fail(BT_ERR_DTYPE, "%s: unsupported y dtype %d", fn, (int)y_dtype);
    BT_TRY(check_ptr(packed, "packed", fn));
    if (N == 0) return ok();
    BT_TRY(check_ptr(x, "x", fn));
    BT_TRY(check_ptr(y, "y", fn));
    hipStream_t s = as_stream(stream);
    if (linear_fuses(N, M, K, x_dtype)) {
        // one launch: every decode workgroup quantizes the tokens into LDS
        const bt::Group g = single_group(packed, M, K, nullptr, nullptr, nullptr, N, y, y_dtype);
        return hip_status(bt::launch_decode_fused(g, x, x_dtype, s), fn);
    }
    const size_t need = linear_ws_bytes(N, K);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(BT_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(BT_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
    uint8_t *b = static_cast<uint8_t *>(workspace);
    int8_t *xq = reinterpret_cast<int8_t *>(b);
    float *xs = reinterpret_cast<float *>(b + align256((size_t)N * (size_t)K));
    int32_t *xsum = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(xs) +
                                                align256((size_t)N * sizeof(float)));
    hipError_t e = bt::launch_quant(x, x_dtype, N, K, xq, xs, xsum, s);
    if (e == hipSuccess) e = run_group(single_group(packed, M, K, xq, xs, xsum, N, y, y_dtype), s);
    return hip_status(e, fn);
}

bt_status bt_ternary_matmul_group(const bt_proj *projs, int count, int64_t K,
                                  const int8_t *xq, const float *x_scale,
                                  const int32_t *x_sum, int64_t N, bt_dtype y_dtype,
                                  bt_stream stream) {
    const char *fn = "bt_ternary_matmul_group";
    if (projs == nullptr || count < 1 || count > BT_MAX_GROUP)
        return fail(BT_ERR_INVALID_ARG, "%s: need 1..%d projections", fn, BT_MAX_GROUP);
    for (int i = 0; i < count; ++i)
        BT_TRY(check_matmul(fn, projs[i].packed, projs[i].M, K, xq, x_scale, x_sum, N,
                            projs[i].y, y_dtype));
    if (N == 0) return ok();
    bt::Group g{};
    g.count = count;
    for (int i = 0; i < count; ++i) g.p[i] = bt::Proj{projs[i].packed, projs[i].M, projs[i].y};
    g.K = K;
    g.xq = xq;
    g.xs = x_scale;
    g.xsum = x_sum;
    g.N = N;
    g.ydt = y_dtype;
    return hip_status(run_group(g, as_stream(stream)), fn);
}

size_t bt_layer_workspace_bytes(const bt_layer *L, int64_t N) {
    if (L == nullptr || N < 0) return 0;
    int64_t Kin[BT_LAYER_INPUTS];
    if (!layer_input_widths(L, Kin)) return 0;
    for (int p = 0; p < BT_LAYER_PROJ; ++p)
        if (check_mk(L->M[p], L->K[p], "bt_layer_workspace_bytes") != BT_OK) return 0;
    ok();
    return carve(Kin, N, nullptr).bytes;
}

}  // extern "C"

namespace bt {

bt_status layer_check(const bt_layer *L, const bt_layer_io *io, const char *fn,
                      size_t *scratch_bytes) {
    if (L == nullptr || io == nullptr)
        return fail(BT_ERR_INVALID_ARG, "%s: layer or io is NULL", fn);
    int64_t Kin[BT_LAYER_INPUTS];
    if (!layer_input_widths(L, Kin))
        return fail(BT_ERR_SHAPE, "%s: q/k/v (or gate/up) have different K", fn);
    const bool base3 = (io->flags & BT_LAYER_BASE3) != 0;
    for (int p = 0; p < BT_LAYER_PROJ; ++p) {
        BT_TRY(base3 ? check_b3(L->M[p], L->K[p], fn) : check_mk(L->M[p], L->K[p], fn));
        BT_TRY(check_ptr(L->w[p], "layer->w[p]", fn));
    }
    const int64_t N = io->N;
    BT_TRY(check_n(N, fn));
    if (io->x_dtype != BT_F32 && io->x_dtype != BT_BF16)
        return fail(BT_ERR_DTYPE, "%s: x dtype must be BT_F32 or BT_BF16", fn);
    if (io->y_dtype != BT_F32 && io->y_dtype != BT_BF16 && io->y_dtype != BT_I32)
        return fail(BT_ERR_DTYPE, "%s: unsupported y dtype %d", fn, (int)io->y_dtype);
    if (io->flags & ~(BT_LAYER_PER_GROUP | BT_LAYER_BASE3))
        return fail(BT_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, (unsigned)io->flags);
    *scratch_bytes = 0;
    if (N == 0) return ok();
    for (int i = 0; i < BT_LAYER_INPUTS; ++i) BT_TRY(check_ptr(io->x[i], "io->x[i]", fn));
    for (int p = 0; p < BT_LAYER_PROJ; ++p) BT_TRY(check_ptr(io->y[p], "io->y[p]", fn));
    *scratch_bytes = carve(Kin, N, nullptr).bytes;
    return ok();
}

// Which kernel runs a block's four groups from 2 tokens on (one launch
// either way, identical results).  The matrix-core decode streams the
// weights once per 16-token group -- the repeats come from the last-level
// cache while the block fits there -- and the prefill kernel once per 64
// tokens, at a higher fixed cost.  Measured per block at 17..127 tokens
// (2B- / 7B- / 13B- / 70B-class blocks: 17 / 51 / 79 / 214 MB of packed
// weights), the decode is the faster up to 6 / 4 / 3 / 2 token groups; e.g.
// 64 tokens of a 70B-class block: 117 us per block on the prefill kernel
// against 195 us on the decode, 96 tokens of 2B-style blocks 31.3 vs 34.1 us
// (at 7 groups the decode wins on blocks streamed from HBM and loses on one
// hot block; from 8 groups the prefill kernel wins).
static bool four_groups_prefill(int64_t N, int64_t packed_bytes) {
    if (N >= BT_PREFILL_MIN_N) return true;
    constexpr int64_t MB = 1 << 20;
    const int64_t max_groups = packed_bytes <= 32 * MB    ? 6
                               : packed_bytes <= 64 * MB  ? 4
                               : packed_bytes <= 128 * MB ? 3
                                                          : 2;
    return (N + 15) / 16 > max_groups;
}

bt_status layer_forward(const bt_layer *L, const bt_layer_io *io, void *workspace,
                        size_t workspace_bytes, bt_stream stream, const char *fn) {
    size_t need_bytes = 0;
    BT_TRY(layer_check(L, io, fn, &need_bytes));
    const int64_t N = io->N;
    if (N == 0) return ok();
    int64_t Kin[BT_LAYER_INPUTS];
    layer_input_widths(L, Kin);
    const bool base3 = (io->flags & BT_LAYER_BASE3) != 0;
    const LayerWs need = carve(Kin, N, nullptr);
    if (workspace == nullptr || workspace_bytes < need.bytes)
        return fail(BT_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need.bytes,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(BT_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);

    hipStream_t s = as_stream(stream);
    if (base3) {
        const bool per_group = (io->flags & BT_LAYER_PER_GROUP) != 0;
        if (!per_group && bt::layer_fusable(Kin, L->M, N, io->x_dtype, true)) {
            const bt::LayerArgs la =
                bt::make_layer_args(L->w, L->M, Kin, io->x, io->y, N, io->y_dtype, true);
            const hipError_t e = bt::launch_layer(la, io->x_dtype, s);
            return e == hipSuccess ? ok() : hip_status(e, fn);
        }
        // the inputs quantized into the workspace (one launch, or one per
        // group before its products), then one base-3 product per projection
        const LayerWs ws = carve(Kin, N, workspace);
        if (!per_group) {
            bt::QuantJobs jobs{};
            for (int i = 0; i < BT_LAYER_INPUTS; ++i) {
                jobs.x[i] = io->x[i];
                jobs.K[i] = Kin[i];
                jobs.xq[i] = ws.xq[i];
                jobs.xs[i] = ws.xs[i];
                jobs.xsum[i] = ws.xsum[i];
            }
            const hipError_t e = bt::launch_quant_jobs(jobs, BT_LAYER_INPUTS, io->x_dtype, N, s);
            if (e != hipSuccess) return hip_status(e, fn);
        }
        static const int kGroupOf[BT_LAYER_PROJ] = {0, 0, 0, 1, 2, 2, 3};
        for (int p = 0; p < BT_LAYER_PROJ; ++p) {
            const int i = kGroupOf[p];
            hipError_t e = hipSuccess;
            if (per_group && (p == 0 || kGroupOf[p - 1] != i))
                e = bt::launch_quant(io->x[i], io->x_dtype, N, Kin[i], ws.xq[i], ws.xs[i],
                                     ws.xsum[i], s);
            if (e == hipSuccess)
                e = bt::launch_b3_gemv(L->w[p], L->M[p], Kin[i], ws.xq[i], ws.xs[i], ws.xsum[i],
                                       N, io->y[p], io->y_dtype, s);
            if (e != hipSuccess) return hip_status(e, fn);
        }
        return ok();
    }
    if (!(io->flags & BT_LAYER_PER_GROUP) && N < BT_PREFILL_MIN_N &&
        bt::layer_fusable(Kin, L->M, N, io->x_dtype)) {
        // one launch for the whole block
        const bt::LayerArgs la = bt::make_layer_args(L->w, L->M, Kin, io->x, io->y, N, io->y_dtype);
        const hipError_t e = bt::launch_layer(la, io->x_dtype, s);
        return e == hipSuccess ? ok() : hip_status(e, fn);
    }
    const LayerWs ws = carve(Kin, N, workspace);
    const bool per_group = (io->flags & BT_LAYER_PER_GROUP) != 0;
    // groups: {q,k,v} <- x0, {o} <- x1, {gate,up} <- x2, {down} <- x3
    static const int kFirst[BT_LAYER_INPUTS] = {0, 3, 4, 6};
    static const int kCount[BT_LAYER_INPUTS] = {3, 1, 2, 1};
    int64_t rows[BT_LAYER_INPUTS];
    for (int i = 0; i < BT_LAYER_INPUTS; ++i) {
        rows[i] = 0;
        for (int j = 0; j < kCount[i]; ++j) rows[i] += L->M[kFirst[i] + j];
    }
    // From 2 tokens on, a block that is not one launch runs its four groups
    // on the matrix cores in one launch (faster than per-group dot4 launches
    // on every block too large for the one-launch kernel: 70B-class at 2
    // tokens 3.37 vs 5.51 ms per 80 blocks, 7B-class at 3 tokens 0.52 vs 1.08
    // ms per 24).  At 1 token each group runs on its own dot4 launch.
    const bool four_groups = N >= 2;
    // The four inputs are all valid at the call: unless asked for per-group
    // launches, the ones that need codes in the workspace are quantized in
    // one launch up front.
    bool quantized = false;
    if (!per_group) {
        bt::QuantJobs jobs{};
        int count = 0;
        for (int i = 0; i < BT_LAYER_INPUTS; ++i) {
            if (!four_groups && bt::decode_fuses_quant(N, rows[i], Kin[i], io->x_dtype)) continue;
            jobs.x[count] = io->x[i];
            jobs.K[count] = Kin[i];
            jobs.xq[count] = ws.xq[i];
            jobs.xs[count] = ws.xs[i];
            jobs.xsum[count] = ws.xsum[i];
            ++count;
        }
        const hipError_t e = bt::launch_quant_jobs(jobs, count, io->x_dtype, N, s);
        if (e != hipSuccess) return hip_status(e, fn);
        quantized = true;
    }
    bt::Group groups[BT_LAYER_INPUTS];
    for (int i = 0; i < BT_LAYER_INPUTS; ++i) {
        bt::Group &g = groups[i];
        g = bt::Group{};
        g.count = kCount[i];
        for (int j = 0; j < g.count; ++j) {
            const int p = kFirst[i] + j;
            g.p[j] = bt::Proj{L->w[p], L->M[p], io->y[p]};
        }
        g.K = Kin[i];
        g.xq = ws.xq[i];
        g.xs = ws.xs[i];
        g.xsum = ws.xsum[i];
        g.N = N;
        g.ydt = io->y_dtype;
    }
    if (quantized && four_groups) {
        // matrix-core decode or prefill: the four groups in one launch
        int64_t bytes = 0;
        for (int p = 0; p < BT_LAYER_PROJ; ++p) bytes += L->M[p] * L->K[p] / 4;
        const hipError_t e = four_groups_prefill(N, bytes)
                                 ? bt::launch_prefill_groups(groups, BT_LAYER_INPUTS, s)
                                 : bt::launch_decode_groups(groups, BT_LAYER_INPUTS, s);
        return e == hipSuccess ? ok() : hip_status(e, fn);
    }
    for (int i = 0; i < BT_LAYER_INPUTS; ++i) {
        const bt::Group &g = groups[i];
        hipError_t e;
        if (N < BT_PREFILL_MIN_N && bt::decode_fuses_quant(N, rows[i], Kin[i], io->x_dtype)) {
            // one launch: the decode kernel quantizes its input itself
            e = bt::launch_decode_fused(g, io->x[i], io->x_dtype, s);
        } else {
            e = quantized ? hipSuccess
                          : bt::launch_quant(io->x[i], io->x_dtype, N, Kin[i], ws.xq[i],
                                             ws.xs[i], ws.xsum[i], s);
            if (e == hipSuccess) e = run_group(g, s);
        }
        if (e != hipSuccess) return hip_status(e, fn);
    }
    return ok();
}

bt_status fail_with(bt_status st, const char *msg) { return fail(st, "%s", msg); }

}  // namespace bt

extern "C" {

bt_status bt_layer_forward(const bt_layer *L, const bt_layer_io *io, bt_stream stream) {
    if (io == nullptr) return fail(BT_ERR_INVALID_ARG, "bt_layer_forward: layer or io is NULL");
    return bt::layer_forward(L, io, io->workspace, io->workspace_bytes, stream,
                             "bt_layer_forward");
}

int bt_layer_one_launch(const bt_layer *L, int64_t N, bt_dtype x_dtype) {
    if (L == nullptr || N < 0 || N > BT_MAX_N) return -1;
    int64_t Kin[BT_LAYER_INPUTS];
    if (!layer_input_widths(L, Kin)) return -1;
    for (int p = 0; p < BT_LAYER_PROJ; ++p)
        if (check_mk(L->M[p], L->K[p], "bt_layer_one_launch") != BT_OK) return -1;
    return N < BT_PREFILL_MIN_N && bt::layer_fusable(Kin, L->M, N, x_dtype) ? 1 : 0;
}

}  // extern "C"
