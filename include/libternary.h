/*
 * libternary.h -- C ABI of the ternary-weight x int8-activation product on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (BitNet b1.58 inference, I2_S-style storage):
 *   - weights are ternary, w in {-1, 0, +1}, stored as 2-bit codes
 *     0, 1, 2 (code = w + 1), four per byte, with one float32 scale per
 *     tensor stored after the codes ([I2S] "Ternary Representation and
 *     Packing", "Per-Tensor Scaling Strategy");
 *   - activations are quantized per token to int8 by absmax ([PARA]
 *     section 5, Quant8 after the AbsMean / RoundClip equations);
 *   - the product is an exact integer sum (the +1 / -1 / 0 = add / subtract /
 *     skip contraction of [PARA] section 5, figure "BitNet b1.58 Ternary
 *     Matrix Multiplication"), dequantized once by weight scale x activation
 *     scale / 127 ([I2S] "How I2_S Kernels Process the Format").
 *
 * Pages cited:
 *   [I2S]  "How BitNet's 1-Bit (I2_S) Quantization Works Compared to Standard
 *          LLM Quantization"
 *   [PARA] "LLM Quantization Paradigms: FP8, AWQ, EXL2 & BitNet b1.58 in 2026"
 *   [PREP] "BitNet Inference Preprocessing: Converting Hugging Face
 *          Checkpoints to I2S GGUF"
 *   [IK]   "ik_llama.cpp 运行 BitNet b1.58 2B 模型实战…"
 *
 * Conventions for every entry point:
 *   - Matrices are row-major.  W is [M, K] = [out, in]; x is [N, K]; y is
 *     [N, M].  N is the number of tokens, 0 <= N <= BT_MAX_N; N = 0 is a
 *     no-op.
 *   - Every array argument is a DEVICE pointer, 16-byte aligned, owned by the
 *     caller.  The library never allocates, frees or synchronizes; scratch
 *     space is passed in by the caller (bt_layer_io.workspace, the workspace
 *     arguments of bt_ternary_linear and bt_quantize_weights), except in
 *     bt_layer_forward_noalloc, whose scratch is a static device array.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously on it; results are ready when the stream is.
 *   - Argument errors are returned synchronously as BT_ERR_* and nothing is
 *     launched.  A failed launch returns BT_ERR_HIP.  A message for the last
 *     error of the calling thread is in bt_last_error().  Faults inside a
 *     kernel surface at the caller's next synchronization, as in HIP.
 *   - Shapes: M % 16 == 0, K % 256 == 0, 0 < K <= 131840 (so that
 *     |sum| <= 127*K < 2^24 converts to float exactly), M > 0.
 *   - Results are deterministic: the integer parts (packed bytes, int8
 *     codes, activation scales, code sums, int32 sums) are exact; float
 *     outputs do not depend on launch order.
 */
#ifndef LIBTERNARY_H
#define LIBTERNARY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BT_ABI_VERSION 8
#define BT_MAX_K 131840
#define BT_MAX_N 2097152 /* tokens per call */
#define BT_TAIL_BYTES 256

typedef enum {
    BT_OK = 0,
    BT_ERR_INVALID_ARG = 1, /* null pointer, negative count, bad enum value */
    BT_ERR_SHAPE = 2,       /* M % 16, K % 256, K range, mismatched shapes */
    BT_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
    BT_ERR_DTYPE = 4,       /* element type not supported for that argument */
    BT_ERR_HIP = 5,         /* a HIP runtime call or launch failed */
    BT_ERR_WORKSPACE = 6    /* workspace missing or smaller than required */
} bt_status;

typedef enum {
    BT_F32 = 0,   /* IEEE binary32 */
    BT_BF16 = 1,  /* bfloat16 (top half of a binary32); outputs are rounded
                     to nearest even from the float32 result */
    BT_I32 = 2    /* outputs only: the raw int32 sum, no dequantization */
} bt_dtype;

typedef void *bt_stream; /* hipStream_t */

/* Version of this ABI (BT_ABI_VERSION of the header it was built from). */
int bt_abi_version(void);

/* Message describing the last error returned on the calling thread
 * (thread-local, valid until the next call on this thread; "" if none). */
const char *bt_last_error(void);

/* ------------------------------------------------------------------------
 * Packed ternary weights ([I2S] "Ternary Representation and Packing",
 * "Per-Tensor Scaling Strategy").
 *
 * Byte layout "T16Q256" (the pages fix the code map and the in-byte order,
 * not the block geometry, which is chosen for 64-lane waves):
 *   W is cut into tiles of 16 rows x 256 columns; tile (m/16, k/256) is the
 *   1024 bytes starting at ((m/16)*(K/256) + k/256) * 1024.  Inside a tile,
 *   slot = (m%16) + 16*((k%64)/16) selects 16 bytes; inside the slot, byte
 *   4*((k%256)/64) + (k%4); inside the byte, group g = (k%16)/4 occupies
 *   bits [7-2g : 6-2g] and holds code = W[m,k] + 1.
 *   So one 16-byte slot read by one lane holds four 32-bit words, each with
 *   the codes of 16 consecutive columns of one row, and a 64-lane wave
 *   reading 16 bytes per lane covers one whole tile.
 *   Bytes [M*K/4, M*K/4+4) hold the float32 scale (little-endian); the
 *   remaining 252 tail bytes are zero.
 * ---------------------------------------------------------------------- */

/* Total size in bytes of a packed M x K matrix: M*K/4 + 256.
 * Returns 0 if the shape is not supported. */
size_t bt_packed_bytes(int64_t M, int64_t K);

/* Pack w[M][K] (int8, values -1/0/+1) and `scale` into `packed`
 * (bt_packed_bytes(M, K) bytes).  A value outside {-1,0,+1} is stored as the
 * nearest state (clamped) and, if `invalid_count` is not NULL, counted: the
 * kernel ADDS the number of such values to *invalid_count (a device int32 the
 * caller zeroes beforehand).  Any M, K with M % 16 == 0 and K % 256 == 0. */
bt_status bt_pack_ternary(const int8_t *w, int64_t M, int64_t K, float scale,
                          uint8_t *packed, int32_t *invalid_count,
                          bt_stream stream);

/* Inverse of bt_pack_ternary: w[M][K] = code - 1.  (The scale stays in the
 * packed tail; read it back with a 4-byte copy from offset M*K/4.) */
bt_status bt_unpack_ternary(const uint8_t *packed, int64_t M, int64_t K,
                            int8_t *w, bt_stream stream);

/* ------------------------------------------------------------------------
 * Float -> ternary weight quantizer, straight into the packed layout
 * ([PARA] section 5, "The Mathematics of BitNet b1.58": the AbsMean
 * quantizer, gamma = mean |W| and RoundClip; [I2S] "Per-Tensor Scaling
 * Strategy": the per-tensor scale max|w|).
 *   s   = mean|W| (BT_WSCALE_ABSMEAN): the exact sum of |W| over all M*K
 *         entries (bf16 widened exactly) divided by M*K and rounded ONCE to
 *         the nearest float32, ties to even -- no summation order can
 *         change it; or max|W| (BT_WSCALE_ABSMAX).
 *   d   = float32(s + eps)   (eps finite and >= 0; the pages leave it open)
 *   W~  = RoundClip(float32(W / d), -1, 1) = max(-1, min(1, round(.)))
 *         with round half to even; 0 / 0 gives 0, nonzero / 0 gives +-1.
 *   packed = the T16Q256 bytes of W~ with d as the tail scale (what
 *         bt_pack_ternary(W~, d) writes), so d * W~ approximates W.
 * w is [M, K] of w_dtype (BT_F32 or BT_BF16) with M * K <= 2^31.  stats, if
 * not NULL, is a device float[2] that receives {s, d}.  workspace is device
 * memory of at least bt_quantize_weights_workspace_bytes() bytes, 16-byte
 * aligned, owned by the caller and used by the call's kernels until they
 * finish (calls that share a workspace must not overlap).  Non-finite
 * weights are outside the contract.  Five launches on `stream`, nothing
 * allocated or synchronized.
 * ---------------------------------------------------------------------- */
#define BT_WSCALE_ABSMEAN 0
#define BT_WSCALE_ABSMAX 1
#define BT_WQ_WORKSPACE_BYTES 4096

size_t bt_quantize_weights_workspace_bytes(void);

bt_status bt_quantize_weights(const void *w, bt_dtype w_dtype, int64_t M, int64_t K,
                              int scale_mode, float eps, uint8_t *packed,
                              float *stats, void *workspace,
                              size_t workspace_bytes, bt_stream stream);

/* ------------------------------------------------------------------------
 * Dequantization (to_float) and the I2_S byte layout.
 * ([IK] section 5.1: an I2_S tensor is dequantized to float32 as a whole
 * before requantization; [I2S] "Ternary Representation and Packing" and
 * "Per-Tensor Scaling Strategy": codes 0/1/2 shifted left by 6 - 2 * group
 * in blocks of QK_I2_S weights, one float scale after the codes.)
 *
 * bt_dequantize_weights: w[m,k] = (code - 1) * scale as a float32 product
 *   (exact: -scale, a signed zero or scale), written as float32, or rounded
 *   to nearest even for BT_BF16.  w is [M, K] row-major.
 *
 * I2_S layout, as read here (the pages do not give QK_I2_S, so it is the
 * caller's `block`: a positive multiple of 4 that divides M*K):
 *   the M*K weights in row-major order are cut into blocks of `block`;
 *   weight j of a block has group g = j / (block/4) and lies in byte
 *   j % (block/4) of the block's block/4 bytes, at bits [7-2g : 6-2g];
 *   the float32 scale follows the M*K/4 code bytes (bt_i2s_bytes(M, K) =
 *   M*K/4 + 4 bytes in all).
 * bt_i2s_import: I2_S bytes -> T16Q256 packed bytes with the same scale.
 *   Code 3 is stored as 2 (+1) and, if invalid_count is not NULL, ADDED to
 *   *invalid_count (a device int32), as bt_pack_ternary does.
 * bt_i2s_export: T16Q256 packed bytes -> I2_S bytes.
 * Shapes as for bt_pack_ternary; buffers are device memory, 16-byte aligned.
 * ---------------------------------------------------------------------- */
size_t bt_i2s_bytes(int64_t M, int64_t K);

bt_status bt_dequantize_weights(const uint8_t *packed, int64_t M, int64_t K,
                                void *w, bt_dtype w_dtype, bt_stream stream);

bt_status bt_i2s_import(const uint8_t *i2s, int64_t M, int64_t K, int64_t block,
                        uint8_t *packed, int32_t *invalid_count,
                        bt_stream stream);

bt_status bt_i2s_export(const uint8_t *packed, int64_t M, int64_t K,
                        int64_t block, uint8_t *i2s, bt_stream stream);

/* ------------------------------------------------------------------------
 * Denser base-3 weight format "B3T1024", 1.625 bits per weight ([IK]
 * sections 5.2, 5.3 and 6: a ternary format of that density over blocks of
 * 64 weights, decoded with integer arithmetic instead of 2-bit masks).  The
 * pages fix the density and the block; the bytes are this library's:
 *   codes c = W + 1; the 64 weights of row m, columns 64i .. 64i+63 are 13
 *   bytes: byte j < 12 = c[4j] + 3c[4j+1] + 9c[4j+2] + 27c[4j+3] + 81c[48+j]
 *   (0..242) and byte 12 = c[60] + 3c[61] + 9c[62] + 27c[63] (0..80), with
 *   c[t] the code of column 64i + t.
 *   Tiles of 16 rows x 1024 columns, 3328 bytes each; tile (m/16, k/1024)
 *   starts at ((m/16)*(K/1024) + k/1024) * 3328.  Lane l = (m%16) +
 *   16*((k%1024)/256) of a tile holds the four blocks b = 0..3 of row m%16,
 *   columns 256*(l/16) + 64b .. of the tile, as 13 32-bit words: words
 *   3b .. 3b+2 hold bytes 0..11 of block b (byte j at word 3b + j/4, byte
 *   j%4) and byte b of word 12 holds byte 12 of block b.  Word d < 12 of lane
 *   l is at tile offset 16*(64*(d/4) + l) + 4*(d%4); word 12 is at
 *   3072 + 4*l.  (A 64-lane wave reads a tile with three 128-bit and one
 *   32-bit coalesced load.)  The float32 scale follows at byte M*K*13/64,
 *   then zeros up to BT_TAIL_BYTES tail bytes.
 * Shapes: M % 16 == 0, K % 1024 == 0, 0 < K <= BT_MAX_K.  Code bytes other
 * than the ones bt_pack_ternary_b3 writes (a byte above 242, or byte 12
 * above 80) are outside the contract.
 *
 * bt_b3_bytes: M*K*13/64 + BT_TAIL_BYTES, or 0 if the shape is not
 *   supported.
 * bt_pack_ternary_b3 / bt_unpack_ternary_b3: as bt_pack_ternary /
 *   bt_unpack_ternary (clamping and counting of values outside {-1,0,+1}
 *   included) for this layout.
 * bt_ternary_gemv_b3: the product of bt_ternary_gemv over B3T1024 weights,
 *   with identical results (the same exact int32 sums and the same float32
 *   dequantization).  Tokens are processed four at a time; every four
 *   tokens stream the weights once.
 * ---------------------------------------------------------------------- */
size_t bt_b3_bytes(int64_t M, int64_t K);

bt_status bt_pack_ternary_b3(const int8_t *w, int64_t M, int64_t K, float scale,
                             uint8_t *packed, int32_t *invalid_count,
                             bt_stream stream);

bt_status bt_unpack_ternary_b3(const uint8_t *packed, int64_t M, int64_t K,
                               int8_t *w, bt_stream stream);

bt_status bt_ternary_gemv_b3(const uint8_t *packed, int64_t M, int64_t K,
                             const int8_t *xq, const float *x_scale,
                             const int32_t *x_sum, int64_t N,
                             void *y, bt_dtype y_dtype, bt_stream stream);

/* ------------------------------------------------------------------------
 * Per-token absmax int8 activation quantization ([PARA] section 5, Quant8).
 *   amax[n] = max_k |x[n,k]| (float32; bf16 inputs are widened exactly)
 *   amax == 0: xq[n,:] = 0, x_scale[n] = 0, x_sum[n] = 0
 *   else     : inv = 127 / amax (float32 division, correctly rounded)
 *              xq[n,k] = clamp(round_half_even(x[n,k] * inv), -127, 127)
 *                        (float32 multiply)
 *              x_scale[n] = amax,  x_sum[n] = sum_k xq[n,k]
 * x is [N, K] of x_dtype (BT_F32 or BT_BF16); xq is int8 [N, K]; x_scale is
 * float32 [N]; x_sum is int32 [N].  Non-finite inputs are outside the
 * contract.
 * ---------------------------------------------------------------------- */
bt_status bt_quant_act(const void *x, bt_dtype x_dtype, int64_t N, int64_t K,
                       int8_t *xq, float *x_scale, int32_t *x_sum,
                       bt_stream stream);

/* ------------------------------------------------------------------------
 * Ternary matrix product with fused dequantization.
 *   acc[n,m] = sum_k W[m,k] * xq[n,k]                      (exact int32)
 *   y[n,m]   = float(acc) * ((s_w * x_scale[n]) / 127)     (float32 ops)
 * where s_w is the scale stored in the packed tail.  y_dtype BT_F32 / BT_BF16
 * writes the dequantized value, BT_I32 writes acc.  xq / x_scale / x_sum are
 * the outputs of bt_quant_act for the same tokens.
 *
 * bt_ternary_gemv is the decode path (few tokens: weights are streamed once
 * from HBM with 128-bit loads, unpacked in registers, and dotted with the
 * int8 activations -- on the int8 matrix cores from 5 tokens, and from 2
 * tokens where the matrix is tall (M >= 4096) or its rows long);
 * bt_ternary_gemm is the prefill path (many tokens: tiled int8 matrix-core
 * product).  Both accept any N >= 0 and return identical results (gemv
 * hands more than 65535 * 16 tokens to the prefill kernel).
 * ---------------------------------------------------------------------- */
bt_status bt_ternary_gemv(const uint8_t *packed, int64_t M, int64_t K,
                          const int8_t *xq, const float *x_scale,
                          const int32_t *x_sum, int64_t N,
                          void *y, bt_dtype y_dtype, bt_stream stream);

bt_status bt_ternary_gemm(const uint8_t *packed, int64_t M, int64_t K,
                          const int8_t *xq, const float *x_scale,
                          const int32_t *x_sum, int64_t N,
                          void *y, bt_dtype y_dtype, bt_stream stream);

/* ------------------------------------------------------------------------
 * Grouped product: up to BT_MAX_GROUP projections that read the same
 * quantized input (q/k/v, or gate/up) in one launch, their 16-row tiles laid
 * end to end in one grid.  This is the GPU form of processing several weight
 * matrices per invocation to cut launch overhead ([I2S] "How I2_S Kernels
 * Process the Format", weight-parallel kernels).  All projections share K;
 * y of projection i is [N, projs[i].M].  The path is chosen from N (decode
 * kernels below BT_PREFILL_MIN_N tokens, the prefill kernel from there on);
 * both give the same bits, so results equal per-projection bt_ternary_gemv /
 * bt_ternary_gemm calls.
 * ---------------------------------------------------------------------- */
#define BT_MAX_GROUP 3
#define BT_PREFILL_MIN_N 128

typedef struct {
    const uint8_t *packed; /* bt_pack_ternary output, M x K */
    int64_t M;
    void *y;               /* [N, M] of y_dtype */
} bt_proj;

bt_status bt_ternary_matmul_group(const bt_proj *projs, int count, int64_t K,
                                  const int8_t *xq, const float *x_scale,
                                  const int32_t *x_sum, int64_t N,
                                  bt_dtype y_dtype, bt_stream stream);

/* ------------------------------------------------------------------------
 * One projection from float activations: the whole BitLinear forward of
 * [PARA] section 5 (Quant8 of the input, the ternary product, the rescale by
 * s_w * x_scale / 127) in one call.  Results are those of bt_quant_act
 * followed by bt_ternary_gemv (N < BT_PREFILL_MIN_N) or bt_ternary_gemm on
 * the same tokens, bit for bit.
 *   x is [N, K] of x_dtype (BT_F32 or BT_BF16), 16-byte aligned; packed, M,
 *   K, y and y_dtype as for bt_ternary_gemv.
 *   - Where the decode kernel can quantize the tokens itself
 *     (bt_linear_one_launch(N, M, K, x_dtype) == 1: 1 token of K up to
 *     32768 in bf16 or 16384 in fp32, 2..4 tokens of short rows) this is
 *     ONE launch: every workgroup rounds the tokens into its LDS, nothing
 *     is written besides y, and the workspace is not touched (it may be
 *     NULL).
 *   - Otherwise the codes, scales and sums go through the workspace
 *     (bt_linear_workspace_bytes(N, K) bytes, 256-byte aligned; a smaller
 *     or missing one gives BT_ERR_WORKSPACE and launches nothing): one
 *     quantization launch, then the product.  Its contents after the call
 *     are unspecified.
 * ---------------------------------------------------------------------- */
size_t bt_linear_workspace_bytes(int64_t N, int64_t K);

/* 1 if bt_ternary_linear runs these arguments as one launch, 0 if as two, -1
 * if they are invalid.  Host-only; no GPU work. */
int bt_linear_one_launch(int64_t N, int64_t M, int64_t K, bt_dtype x_dtype);

bt_status bt_ternary_linear(const uint8_t *packed, int64_t M, int64_t K,
                            const void *x, bt_dtype x_dtype, int64_t N,
                            void *y, bt_dtype y_dtype, void *workspace,
                            size_t workspace_bytes, bt_stream stream);

/* ------------------------------------------------------------------------
 * Per-layer projection driver.  One transformer block has seven ternary
 * projections ([PREP] "Stage 1": q, k, v, o, gate, up, down).  They are run
 * as four dependent groups that share a quantized input:
 *   x[0] (attention input)  -> q, k, v      (K[0] == K[1] == K[2])
 *   x[1] (attention output) -> o            (K[3])
 *   x[2] (FFN input)        -> gate, up     (K[4] == K[5])
 *   x[3] (FFN hidden)       -> down         (K[6])
 * Each group quantizes its input once (bt_quant_act semantics) and runs its
 * projections; the path (decode or prefill) is chosen from N.  Outputs are
 * identical to calling bt_quant_act followed by bt_ternary_gemv /
 * bt_ternary_gemm per projection, whatever the launch structure:
 *   - 1..4 tokens, every K >= 2048, the codes of all four inputs within
 *     128 KiB, 8-element input chunks within 8 per thread of a 1024-thread
 *     workgroup, and from 2 tokens on at most 64 / 20 / 12 MB of packed
 *     weights at 2 / 3 / 4 tokens (beyond that the matrix-core launch below
 *     is faster) -- e.g. 1 token of an 8192/28672 block, up to 3 of a
 *     2560/6912 block: ONE launch for the whole block.  The kernel
 *     quantizes all four inputs in its prologue and streams the seven
 *     weight matrices back to back ([PREP] "Stage 1" lists them), so the
 *     four inputs must all be valid when the call is made -- which is what
 *     this interface takes.  The workspace is not touched.
 *   - otherwise, from 2 tokens on: one launch that quantizes the four
 *     inputs into the workspace, then one matrix-core launch for all four
 *     groups: the decode kernel (weights streamed once per 16 tokens) up to
 *     6 / 4 / 3 / 2 groups of 16 tokens for blocks of at most 32 / 64 / 128
 *     MiB / more of packed weights, the prefill kernel (once per 64 tokens)
 *     beyond that and from BT_PREFILL_MIN_N tokens on (measured crossovers;
 *     the two give the same bits).
 *   - otherwise (1 token of a block too large for one launch): one decode
 *     launch per group, each quantizing its own input in its prologue where
 *     the row fits (the other inputs are quantized by one launch first).
 *   - with BT_LAYER_PER_GROUP in io->flags: the groups one after the other,
 *     each quantizing its own input (in the decode kernel, or by a launch of
 *     its own) before its product -- the order of a decoder whose inputs
 *     are produced between groups.
 *   The workspace's contents after the call are unspecified.
 * ---------------------------------------------------------------------- */
#define BT_LAYER_PROJ 7
#define BT_LAYER_INPUTS 4

typedef struct {
    const uint8_t *w[BT_LAYER_PROJ]; /* packed q,k,v,o,gate,up,down */
    int64_t M[BT_LAYER_PROJ];
    int64_t K[BT_LAYER_PROJ];
} bt_layer;

typedef struct {
    int64_t N;                          /* tokens */
    const void *x[BT_LAYER_INPUTS];     /* [N, K of its group], x_dtype */
    bt_dtype x_dtype;                   /* BT_F32 or BT_BF16 */
    void *y[BT_LAYER_PROJ];             /* [N, M[p]], y_dtype */
    bt_dtype y_dtype;                   /* BT_F32, BT_BF16 or BT_I32 */
    void *workspace;                    /* device scratch, 256-byte aligned */
    size_t workspace_bytes;             /* >= bt_layer_workspace_bytes() */
    uint32_t flags;                     /* 0, BT_LAYER_PER_GROUP, BT_LAYER_BASE3 */
} bt_layer_io;

/* io->flags: run the four groups as four launches even where one would do. */
#define BT_LAYER_PER_GROUP 1u
/* The seven weight pointers hold base-3 B3T1024 bytes (bt_pack_ternary_b3;
 * every K a multiple of 1024).  Results are those of the T16Q256 path on the
 * same weights.  1..2 tokens with every K >= 4096 and N * (sum of the four
 * input widths) <= 80 KiB (e.g. 1 token of an 8192/28672 block) run as ONE
 * launch, as above, with the base-3 decode; otherwise the inputs are
 * quantized into the workspace and each projection is a bt_ternary_gemv_b3
 * product. */
#define BT_LAYER_BASE3 2u

/* Scratch needed by bt_layer_forward for N tokens (quantized inputs, their
 * scales and sums).  Returns 0 if the layer's shapes are invalid. */
size_t bt_layer_workspace_bytes(const bt_layer *layer, int64_t N);

bt_status bt_layer_forward(const bt_layer *layer, const bt_layer_io *io,
                           bt_stream stream);

/* ------------------------------------------------------------------------
 * Allocation-free per-layer driver.  For callers that cannot allocate device
 * memory or hand in a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.
 *
 * bt_layer_forward_noalloc runs exactly what bt_layer_forward runs for the
 * same layer and io, with identical results; io->workspace and
 * io->workspace_bytes are ignored.  The scratch those kernels use (the
 * quantized inputs, their scales and sums: bt_layer_workspace_bytes(layer,
 * io->N) bytes) is a static device array of BT_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends (32 MiB:
 * e.g. 2048 tokens of a 2560/6912 block need 29.9 MB, 8 tokens of an
 * 8192/28672 block 0.43 MB, 1..4 tokens of a one-launch block none).
 *   - A call that needs more returns BT_ERR_WORKSPACE and launches nothing;
 *     every other argument error is reported as by bt_layer_forward.
 *   - Nothing is allocated, freed or synchronized.  The first call on a GPU
 *     looks up the array's address there (hipGetSymbolAddress); later calls
 *     reuse it.
 *   - Every call on one GPU uses that GPU's array.  Calls ordered on one
 *     stream are safe; calls that overlap on one GPU (other streams, other
 *     host threads without ordering) race and their results are undefined.
 * ---------------------------------------------------------------------- */
#define BT_NOALLOC_SCRATCH_BYTES (32u << 20)

bt_status bt_layer_forward_noalloc(const bt_layer *layer, const bt_layer_io *io,
                                   bt_stream stream);

/* 1 if bt_layer_forward runs this layer of T16Q256 weights for N tokens of
 * x_dtype as one launch (io->flags 0), 0 if as per-group launches, -1 if the
 * layer or the arguments are invalid.  Host-only; no GPU work. */
int bt_layer_one_launch(const bt_layer *layer, int64_t N, bt_dtype x_dtype);

#ifdef __cplusplus
}
#endif

#endif /* LIBTERNARY_H */
