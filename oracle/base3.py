"""CPU oracle for the denser base-3 packing ("B3": 64 weights in 13 bytes).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite, the
package smoke check and the benchmark's CPU-baseline leg are its only callers.

What the pages fix ("ik_llama.cpp 运行 BitNet b1.58 2B 模型实战…", sections 5.2,
5.3 and 6): a 1.625-bit-per-weight ternary format works on blocks of 64
weights (the column count must be a multiple of 64) and is decoded with
multiplies, adds and shifts.  1.625 bits x 64 = 104 bits = 13 bytes.  The
byte encoding is not given; this one is ours:

  codes c = w + 1 in {0, 1, 2} (the code map of the 2-bit format);
  block of 64 columns, byte j = 0..11 holds
      c[4j] + 3 c[4j+1] + 9 c[4j+2] + 27 c[4j+3] + 81 c[48+j]   (0..242)
  and byte 12 holds
      c[60] + 3 c[61] + 9 c[62] + 27 c[63]                       (0..80);
  so byte j's low four base-3 digits are columns 4j..4j+3 in order (one
  int8x4 word after decoding) and its fifth digit is column 48 + j.

Matrix layout "B3T1024": W [M, K] with M % 16 == 0 and K % 1024 == 0 is cut
into tiles of 16 rows x 1024 columns, tile (m/16, k/1024) at byte offset
((m/16) * (K/1024) + k/1024) * 3328.  Lane l = r + 16 s (r = m % 16, s =
(k % 1024) / 256) owns the 4 blocks (52 bytes, 13 little-endian 32-bit words)
of row r, columns 256 s .. 256 s + 255 of the tile, block b = columns
256 s + 64 b .. 256 s + 64 b + 63.  Words 3b, 3b+1, 3b+2 hold bytes 0..11 of
block b (byte j in word 3b + j // 4 at byte j % 4); word 12 holds byte 12 of
block b at its byte b.  Word d < 12 of lane l sits at tile offset
16 (64 (d // 4) + l) + 4 (d % 4) -- so words 0..11 are three 16-byte chunks
that a 64-lane wave reads with three fully coalesced 128-bit loads -- and
word 12 at tile offset 3072 + 4 l.  The float32 scale follows the
M * K * 13 / 64 code bytes, then zeros up to 256 tail bytes.
"""
from __future__ import annotations

import numpy as np

TILE_ROWS, TILE_COLS, TILE_BYTES = 16, 1024, 3328


def packed_bytes(M: int, K: int) -> int:
    if M % TILE_ROWS or K % TILE_COLS:
        raise ValueError("B3 needs M % 16 == 0 and K % 1024 == 0")
    return M * K * 13 // 64 + 256


def encode_block(c: np.ndarray) -> np.ndarray:
    """64 codes (0..2) -> 13 bytes."""
    c = np.asarray(c, dtype=np.int64).reshape(64)
    out = np.empty(13, dtype=np.uint8)
    for j in range(12):
        out[j] = (c[4 * j] + 3 * c[4 * j + 1] + 9 * c[4 * j + 2] + 27 * c[4 * j + 3]
                  + 81 * c[48 + j])
    out[12] = c[60] + 3 * c[61] + 9 * c[62] + 27 * c[63]
    return out


def decode_block(b: np.ndarray) -> np.ndarray:
    """13 bytes -> 64 codes (0..2)."""
    b = np.asarray(b, dtype=np.int64).reshape(13)
    c = np.empty(64, dtype=np.int64)
    for j in range(12):
        v = b[j]
        for i in range(4):
            c[4 * j + i] = (v // 3 ** i) % 3
        c[48 + j] = v // 81
    for i in range(4):
        c[60 + i] = (b[12] // 3 ** i) % 3
    return c


def _lane_runs(M: int, K: int, rows=None):
    """(row, first column, byte offsets of the 52 bytes of the lane's four
    blocks in block order) of every lane (of the given rows only, if rows is
    not None)."""
    qt = K // TILE_COLS
    keep = None if rows is None else set(int(r) for r in rows)
    for mt in range(M // TILE_ROWS):
        for q in range(qt):
            base = (mt * qt + q) * TILE_BYTES
            for lane in range(64):
                r, s = lane % 16, lane // 16
                if keep is not None and mt * TILE_ROWS + r not in keep:
                    continue
                offs = []
                for b in range(4):       # run byte 13 b + j = byte j of block b
                    for j in range(13):
                        d, t = (3 * b + j // 4, j % 4) if j < 12 else (12, b)
                        word = 16 * (64 * (d // 4) + lane) + 4 * (d % 4) if d < 12 \
                            else 3072 + 4 * lane
                        offs.append(base + word + t)
                yield mt * TILE_ROWS + r, q * TILE_COLS + 256 * s, offs


def pack(w: np.ndarray, scale: float) -> np.ndarray:
    """int8 ternary W [M, K] -> B3T1024 bytes (codes, scale, zero tail)."""
    w = np.asarray(w, dtype=np.int8)
    if w.min(initial=0) < -1 or w.max(initial=0) > 1:
        raise ValueError("weights must be -1, 0 or +1")
    M, K = w.shape
    out = np.zeros(packed_bytes(M, K), dtype=np.uint8)
    codes = w.astype(np.int64) + 1
    for row, col, offs in _lane_runs(M, K):
        run = np.concatenate([encode_block(codes[row, col + 64 * b: col + 64 * b + 64])
                              for b in range(4)])
        out[offs] = run
    n = M * K * 13 // 64
    out[n: n + 4] = np.array([scale], np.float32).view(np.uint8)
    return out


def unpack(buf: np.ndarray, M: int, K: int, rows=None):
    """B3T1024 bytes -> (int8 W [M, K] -- or [len(rows), K] for the given
    rows -- and the float32 scale)."""
    buf = np.asarray(buf, dtype=np.uint8)
    order = None if rows is None else {int(r): i for i, r in enumerate(rows)}
    w = np.empty((M if rows is None else len(rows), K), dtype=np.int8)
    for row, col, offs in _lane_runs(M, K, rows):
        run = buf[offs]
        dst = row if order is None else order[row]
        for b in range(4):
            w[dst, col + 64 * b: col + 64 * b + 64] = decode_block(run[13 * b: 13 * b + 13]) - 1
    n = M * K * 13 // 64
    return w, np.float32(buf[n: n + 4].copy().view(np.float32)[0])
