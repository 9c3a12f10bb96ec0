/*
 * bt_oracle.c -- plain CPU oracle for the ternary-weight x int8-activation
 * product (BitNet b1.58, I2_S-style storage).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or
 * calls this file, and this file includes nothing of the GPU library.  Only
 * the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg load it.
 *
 * Every function is the plain definition written out, one element at a time,
 * so that it can be checked by eye against the sources below.  Nothing is
 * blocked, fused or reordered.  The optional OpenMP pragmas only split the
 * outermost loop over independent output rows.
 *
 * Sources (web pages; cited by title and section):
 *   [I2S]   "How BitNet's 1-Bit (I2_S) Quantization Works Compared to
 *           Standard LLM Quantization" (instagit.com).
 *   [PARA]  "LLM Quantization Paradigms: FP8, AWQ, EXL2 & BitNet b1.58 in
 *           2026" (gujjufanclub.com).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp
 *        -shared -fPIC   (no -march=native, no -ffast-math: the float steps
 *        below must be plain IEEE binary32 / binary64 operations).
 *
 * Readings of the pages that this file depends on (each is also listed with
 * its justification in the design notes of the repository):
 *   R1  code = w + 1, so {-1,0,+1} -> {0,1,2}; code 3 is never written.
 *       [I2S] "Ternary Representation and Packing" gives the three states
 *       and their 2-bit integers 0,1,2 in that order.
 *   R2  Within a byte, group g sits at bits [7-2g : 6-2g] (group 0 in the
 *       two most significant bits).  [I2S] "Ternary Representation and
 *       Packing" shifts a code left by (6 - 2*group).
 *   R3  The tiling of rows and columns onto bytes ("T16Q256") is chosen for
 *       the GPU, since the pages do not state the block size; see
 *       bto_byte_index() for the whole definition.
 *   R4  One fp32 scale follows the packed codes at byte offset M*K/4
 *       ([I2S] "Per-Tensor Scaling Strategy"); the buffer is padded with
 *       zero bytes to M*K/4 + 256.
 *   R5  Quant8 is per-token absmax to int8 ([PARA] section 5, the
 *       activation-quantization sentence after the RoundClip equation).
 *       The formula is not printed.  Reading: amax = max|x| in binary32;
 *       inv = 127 / amax (binary32 division, correctly rounded);
 *       xq = clamp(round-half-even(x * inv), -127, 127) with a binary32
 *       multiply; the token's scale is amax; amax == 0 gives xq = 0 and
 *       scale 0.  When amax is so small (below 127 / FLT_MAX) that 127 / amax
 *       overflows, the same binary32 steps are kept with inv = +infinity:
 *       x * inv is +-infinity for x != 0, which the clamp turns into
 *       127 * sign(x), and the one undefined product, 0 * infinity (NaN in
 *       IEEE arithmetic), is defined here as 0.  This is a convention for
 *       inputs the pages never consider, not the real-number value of
 *       x * 127 / amax (for x = 2e-38, amax = 1e-37 that is 25.4, while this
 *       gives 127).
 *   R6  The contraction is carried out in integers and dequantized once:
 *       y = acc * s_w * s_a / 127 ([I2S] "How I2_S Kernels Process the
 *       Format" multiplies by the shared per-tensor scale; a per-tensor
 *       scale factors out of the sum).
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------- */
/* Layout (R3, R4)                                                        */
/* ---------------------------------------------------------------------- */

/* Size in bytes of a packed M x K ternary matrix: M*K/4 bytes of 2-bit codes
 * (four codes per byte, [I2S] "Ternary Representation and Packing") followed
 * by a 256-byte tail that starts with the fp32 scale (R4). */
int64_t bto_packed_bytes(int64_t M, int64_t K)
{
    return M * K / 4 + 256;
}

/* Byte that holds W[m,k] and the bit shift of its 2-bit field.
 *
 * The matrix is cut into tiles of 16 rows x 256 columns.  Tile (mt, q)
 * (mt = m/16, q = k/256) occupies 1024 consecutive bytes; tiles are stored
 * row-tile major: tile index mt*(K/256) + q.  Inside a tile, 64 slots of
 * 16 bytes; slot = r + 16*h where r = m%16 and h = (k%64)/16.  Inside a slot,
 * byte 4*t + i with t = (k%256)/64 and i = k%4.  Inside the byte, group
 * g = (k%16)/4 sits at bits [7-2g : 6-2g] (R2).
 */
static void bto_byte_index(int64_t m, int64_t k, int64_t K,
                           int64_t *byte, int *shift)
{
    int64_t mt = m / 16, r = m % 16;
    int64_t q = k / 256;
    int64_t t = (k % 256) / 64;
    int64_t h = (k % 64) / 16;
    int64_t g = (k % 16) / 4;
    int64_t i = k % 4;
    int64_t slot = r + 16 * h;
    *byte = ((mt * (K / 256) + q) * 64 + slot) * 16 + 4 * t + i;
    *shift = (int)(6 - 2 * g);
}

/* Pack an int8 ternary matrix w[M][K] (row-major) with per-tensor scale.
 * Values outside {-1,0,+1} are clamped to the nearest state and counted.
 * Returns the number of such values.  Requires M%16 == 0 and K%256 == 0. */
int64_t bto_pack(const int8_t *w, int64_t M, int64_t K, float scale,
                 uint8_t *out)
{
    int64_t data = M * K / 4;
    int64_t invalid = 0;
    memset(out, 0, (size_t)bto_packed_bytes(M, K));
    #pragma omp parallel for reduction(+:invalid) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            int v = w[m * K + k];
            if (v < -1) { v = -1; ++invalid; }
            if (v > 1)  { v = 1;  ++invalid; }
            unsigned code = (unsigned)(v + 1);          /* R1 */
            int64_t byte; int shift;
            bto_byte_index(m, k, K, &byte, &shift);
            out[byte] |= (uint8_t)(code << shift);      /* R2 */
        }
    }
    memcpy(out + data, &scale, sizeof(float));          /* R4 */
    return invalid;
}

/* Read one weight back: the 2-bit code at W[m,k], minus one (R1). */
static int bto_weight(const uint8_t *packed, int64_t m, int64_t k, int64_t K)
{
    int64_t byte; int shift;
    bto_byte_index(m, k, K, &byte, &shift);
    int code = (packed[byte] >> shift) & 3;
    return code - 1;
}

/* Unpack to int8 w[M][K] in {-1,0,+1} (a code of 3 would give +2, which the
 * tests treat as a corrupt buffer). */
void bto_unpack(const uint8_t *packed, int64_t M, int64_t K, int8_t *w)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            w[m * K + k] = (int8_t)bto_weight(packed, m, k, K);
}

/* The per-tensor scale stored after the codes (R4). */
float bto_scale(const uint8_t *packed, int64_t M, int64_t K)
{
    float s;
    memcpy(&s, packed + M * K / 4, sizeof(float));
    return s;
}

/* ---------------------------------------------------------------------- */
/* Per-token absmax activation quantization (R5)                          */
/* ---------------------------------------------------------------------- */

/* One token: x[0..K) in binary32. */
static void bto_quant_token(const float *x, int64_t K,
                            int8_t *xq, float *scale, int32_t *sum)
{
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = fabsf(x[k]);
        if (a > amax) amax = a;
    }
    int64_t s = 0;
    if (amax == 0.0f) {
        for (int64_t k = 0; k < K; ++k) xq[k] = 0;
        *scale = 0.0f;
        *sum = 0;
        return;
    }
    float inv = 127.0f / amax;               /* binary32, correctly rounded */
    for (int64_t k = 0; k < K; ++k) {
        float p = x[k] * inv;                /* binary32 product */
        if (isinf(inv) && x[k] == 0.0f) p = 0.0f;  /* R5: 0 * inf := 0 */
        float r = rintf(p);                  /* round half to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        xq[k] = (int8_t)r;
        s += xq[k];
    }
    *scale = amax;
    *sum = (int32_t)s;
}

void bto_quant_act_f32(const float *x, int64_t N, int64_t K,
                       int8_t *xq, float *scale, int32_t *sum)
{
    for (int64_t n = 0; n < N; ++n)
        bto_quant_token(x + n * K, K, xq + n * K, scale + n, sum + n);
}

/* bfloat16 input: each value is the top 16 bits of a binary32, so widening
 * is exact. */
void bto_quant_act_bf16(const uint16_t *x, int64_t N, int64_t K,
                        int8_t *xq, float *scale, int32_t *sum)
{
    float *row = (float *)malloc((size_t)K * sizeof(float));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            uint32_t u = (uint32_t)x[n * K + k] << 16;
            memcpy(&row[k], &u, sizeof(float));
        }
        bto_quant_token(row, K, xq + n * K, scale + n, sum + n);
    }
    free(row);
}

/* ---------------------------------------------------------------------- */
/* Integer product and dequantization (R6)                                */
/* ---------------------------------------------------------------------- */

/* acc[n][j] = sum_k W[rows[j], k] * xq[n][k], for j < nrows, in int64 and
 * checked to fit int32.  rows == NULL means every row (nrows = M, j = m).
 * W is read through the packed layout one element at a time.  Output is
 * [N][nrows] row-major.  Returns 0, or 1 if some sum does not fit int32. */
int bto_matmul_i32(const uint8_t *packed, int64_t M, int64_t K,
                   const int64_t *rows, int64_t nrows,
                   const int8_t *xq, int64_t N, int32_t *acc)
{
    int overflow = 0;
    if (rows == NULL) nrows = M;
    #pragma omp parallel for reduction(|:overflow) schedule(dynamic, 4)
    for (int64_t j = 0; j < nrows; ++j) {
        int64_t m = rows ? rows[j] : j;
        int8_t *wrow = (int8_t *)malloc((size_t)K);
        for (int64_t k = 0; k < K; ++k)
            wrow[k] = (int8_t)bto_weight(packed, m, k, K);
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)wrow[k] * (int64_t)xq[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
            acc[n * nrows + j] = (int32_t)s;
        }
        free(wrow);
    }
    return overflow;
}

/* y[n][j] = acc[n][j] * s_w * s_a[n] / 127, in binary64. */
void bto_dequant(const int32_t *acc, int64_t N, int64_t ncols, double s_w,
                 const float *s_a, double *y)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < ncols; ++j)
            y[n * ncols + j] =
                (double)acc[n * ncols + j] * s_w * (double)s_a[n] / 127.0;
}
