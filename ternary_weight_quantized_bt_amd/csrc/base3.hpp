// base3.hpp -- decode side of the base-3 weight format "B3T1024" (64 ternary
// weights in 13 bytes, 1.625 bits per weight), shared by the per-matrix
// decode kernel (base3.hip) and the per-layer kernel (layer.hip).
//
// [IK] "ik_llama.cpp 运行 BitNet b1.58 2B 模型实战…", sections 5.2, 5.3 and 6:
// a 1.625-bit ternary format over blocks of 64 weights, decoded with integer
// arithmetic rather than 2-bit masks.  The encoding and the tile layout are
// this library's (libternary.h defines both).
//
// GPU decode.  A byte's four low base-3 digits are the codes of four
// consecutive columns -- one int8x4 dot operand -- and its fifth digit is the
// code of one of columns 48..59.  Rather than divide, every workgroup builds a
// table in LDS: entry v holds the four low digits of v as bytes and, in a
// second word, the fifth digit v / 81 repeated in all four bytes.  One 8-byte
// LDS read per weight byte yields a dot operand ready to use, and the fifth
// digits of four bytes are merged into the operand of columns 48+4g..51+4g
// with two byte permutes and an or.  The table is stored 32 times over (lane l
// reads copy l % 32 at byte v * 256 + 8 (l % 32)), so any 32 lanes served
// together hit 32 distinct 8-byte bank pairs whatever the weights are: table
// lookups without bank conflicts.  Per 64 weights a lane spends 13 byte
// permutes (the table address of each byte), 13 LDS reads, 9 merge operations
// and 16 dot4 per token (the 2-bit decode: 20 bit operations and 16 dot4).

#pragma once

#include "common.hpp"

namespace bt {

constexpr int kB3Cols = 1024;        // columns of one B3 tile
constexpr int kB3TileBytes = 3328;   // 16 x 1024 codes at 1.625 bits
constexpr int kB3Copies = 32;        // table copies (lane % 32)
constexpr int kB3TabBytes = 256 * kB3Copies * 8;  // every byte value, 8 bytes per entry

__host__ __device__ inline int64_t b3_code_bytes(int64_t M, int64_t K) { return M * K / 64 * 13; }

// The four low base-3 digits of a byte as four bytes (codes, 0..2).
__device__ __forceinline__ uint32_t low_digits(uint32_t v) {
    return (v % 3) | ((v / 3 % 3) << 8) | ((v / 9 % 3) << 16) | ((v / 27 % 3) << 24);
}

// Builds the decode table in LDS (kB3TabBytes at tab): thread t of n computes
// entry v = t / 4 once and writes copies 8 (t % 4) .. 8 (t % 4) + 7, 64
// contiguous bytes at v * 256 + 64 (t % 4).  Byte values above 242 (never
// written by the encoder) decode to zeros.
__device__ __forceinline__ void b3_build_table(uint8_t *tab, int tid, int n) {
    for (int t = tid; t < 256 * 4; t += n) {
        const uint32_t v = (uint32_t)t / 4;
        const uint32_t lo = v < 243 ? low_digits(v) : 0u;
        const uint32_t hi = v < 243 ? (v / 81) * 0x01010101u : 0u;
        v4u *dst = reinterpret_cast<v4u *>(tab + 64 * t);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = v4u{lo, hi, lo, hi};
    }
}

// One lane's share of one tile: 13 words.
struct B3Slot {
    v4u c0, c1, c2;
    uint32_t last;
};

// NT: non-temporal loads (each byte is read once).
template <bool NT = false>
__device__ __forceinline__ B3Slot load_slot(const uint8_t *tile, int lane) {
    const gptr<const v4u> p = to_global(reinterpret_cast<const v4u *>(tile)) + lane;
    const gptr<const uint32_t> w = to_global(reinterpret_cast<const uint32_t *>(tile + 3072)) + lane;
    B3Slot s;
    if (NT) {
        s.c0 = __builtin_nontemporal_load(p);
        s.c1 = __builtin_nontemporal_load(p + 64);
        s.c2 = __builtin_nontemporal_load(p + 128);
        s.last = __builtin_nontemporal_load(w);
    } else {
        s.c0 = p[0];
        s.c1 = p[64];
        s.c2 = p[128];
        s.last = *w;
    }
    return s;
}

// Table entry of byte i of `word` for this lane: {low digits, fifth digit x 4}.
// v_perm_b32 builds the LDS byte address v * 256 + l8 in one instruction:
// result byte 0 = byte 0 of l8, result byte 1 = byte i of word, bytes 2, 3 = 0.
__device__ __forceinline__ uint2 lookup(const uint8_t *tab, uint32_t word, int i, uint32_t l8) {
    const uint32_t addr = __builtin_amdgcn_perm(word, l8, 0x0C0C0000u | ((4u + i) << 8));
    return *reinterpret_cast<const uint2 *>(tab + addr);
}

// Byte i of the result from byte 0 of hi (each hi holds one value in all
// four bytes): two byte permutes and an or.
__device__ __forceinline__ uint32_t merge4(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3) {
    const uint32_t lo = __builtin_amdgcn_perm(h1, h0, 0x0C0C0400u);  // h0 h1 0 0
    const uint32_t hi = __builtin_amdgcn_perm(h3, h2, 0x04000C0Cu);  // 0 0 h2 h3
    return lo | hi;
}

// Adds sum_k code[k] * x[n, k] over the lane's 256 columns of one tile for
// tokens n < nvalid.  x points at the lane's first column of token 0; token
// rows are K bytes apart.
template <int NT>
__device__ __forceinline__ void b3_dot(const B3Slot &sl, const uint8_t *tab, uint32_t l8,
                                       const int8_t *x, int64_t K, int nvalid, int acc[NT]) {
    const uint32_t w[13] = {sl.c0.x, sl.c0.y, sl.c0.z, sl.c0.w, sl.c1.x, sl.c1.y, sl.c1.z,
                            sl.c1.w, sl.c2.x, sl.c2.y, sl.c2.z, sl.c2.w, sl.last};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint2 e[12];
#pragma unroll
        for (int j = 0; j < 12; ++j) e[j] = lookup(tab, w[3 * b + j / 4], j % 4, l8);
        const uint32_t e12 = lookup(tab, w[12], b, l8).x;
        uint32_t d[3];
#pragma unroll
        for (int g = 0; g < 3; ++g)
            d[g] = merge4(e[4 * g].y, e[4 * g + 1].y, e[4 * g + 2].y, e[4 * g + 3].y);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if (n >= nvalid) break;
            const uint4 *xv = reinterpret_cast<const uint4 *>(x + n * K + 64 * b);
            const uint4 a0 = xv[0], a1 = xv[1], a2 = xv[2], a3 = xv[3];
            const uint32_t xa[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                                     a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
            int s = acc[n];
#pragma unroll
            for (int j = 0; j < 12; ++j) s = __builtin_amdgcn_sdot4((int)e[j].x, (int)xa[j], s, false);
#pragma unroll
            for (int g = 0; g < 3; ++g) s = __builtin_amdgcn_sdot4((int)d[g], (int)xa[12 + g], s, false);
            acc[n] = __builtin_amdgcn_sdot4((int)e12, (int)xa[15], s, false);
        }
    }
}

}  // namespace bt
