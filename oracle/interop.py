"""CPU oracle for dequantization (to_float) and the I2_S byte layout.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite, the
package smoke check and the benchmark's CPU-baseline leg are its only callers.

What it computes, cited by page title and section:
  [I2S]  "How BitNet's 1-Bit (I2_S) Quantization Works Compared to Standard
         LLM Quantization", "Ternary Representation and Packing": the states
         -1, 0, +1 are the 2-bit codes 0, 1, 2, and a code is shifted left by
         6 - 2 * group inside its byte; the block size QK_I2_S of that
         formula is not given.  "Per-Tensor Scaling Strategy": one float
         scale after the quantized data.
  [IK]   "ik_llama.cpp 运行 BitNet b1.58 2B 模型实战…", section 5.1 (why
         --allow-requantize is needed): an I2_S tensor is turned back into
         float32 as a whole (to_float) before it is requantized.

Readings (the pages leave these open):
  I1  An I2_S buffer holds the M*K weights in row-major order, cut into
      blocks of `block` consecutive weights (the pages' QK_I2_S, left to
      the caller: a multiple of 4 that divides M*K).  A block owns
      block/4 bytes; weight j of the block has group g = j // (block/4)
      and sits in byte j % (block/4) of the block, at bits [7-2g : 6-2g].
  I2  The float32 scale follows the M*K/4 code bytes directly (M*K/4 + 4
      bytes in all, little-endian).
  I3  Code 3 is never written; on import it counts as invalid and is read
      as +1 (the packer's clamp).
  I4  to_float: w = (code - 1) * scale, exact in float32; a bfloat16 output
      is that float32 rounded to nearest even.
"""
from __future__ import annotations

import numpy as np


def i2s_bytes(M: int, K: int) -> int:
    return M * K // 4 + 4


def _check_block(n: int, block: int):
    if block <= 0 or block % 4 or n % block:
        raise ValueError(f"block must be a positive multiple of 4 dividing {n}")


def i2s_pack(w: np.ndarray, scale: float, block: int) -> np.ndarray:
    """int8 ternary w [M, K] -> I2_S bytes (codes, then the float32 scale)."""
    w = np.asarray(w, dtype=np.int8)
    if w.min(initial=0) < -1 or w.max(initial=0) > 1:
        raise ValueError("weights must be -1, 0 or +1")
    n = w.size
    _check_block(n, block)
    q = block // 4
    codes = (w.ravel().astype(np.int16) + 1).astype(np.uint8).reshape(n // block, 4, q)
    out = np.zeros((n // block, q), dtype=np.uint8)
    for g in range(4):  # group g: weights g*q .. g*q + q - 1 of every block
        out |= codes[:, g, :] << np.uint8(6 - 2 * g)
    return np.concatenate([out.ravel(), np.array([scale], np.float32).view(np.uint8)])


def i2s_unpack(buf: np.ndarray, M: int, K: int, block: int):
    """I2_S bytes -> (int8 w [M, K], float32 scale, count of code-3 values)."""
    n = M * K
    _check_block(n, block)
    buf = np.asarray(buf, dtype=np.uint8)
    q = block // 4
    b = buf[: n // 4].reshape(n // block, q)
    codes = np.empty((n // block, 4, q), dtype=np.uint8)
    for g in range(4):
        codes[:, g, :] = (b >> np.uint8(6 - 2 * g)) & np.uint8(3)
    codes = codes.ravel()
    invalid = int(np.count_nonzero(codes == 3))
    codes = np.minimum(codes, 2)
    scale = buf[n // 4: n // 4 + 4].copy().view(np.float32)[0]
    return (codes.astype(np.int8) - 1).reshape(M, K), np.float32(scale), invalid


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even
    (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def to_float(w: np.ndarray, scale: float, dtype: str = "f32") -> np.ndarray:
    """Dequantized weights (reading I4) from the ternary values w and the
    tensor scale: float32, or bfloat16 bit patterns as uint16."""
    y = np.asarray(w, dtype=np.float32) * np.float32(scale)
    if dtype == "f32":
        return y
    if dtype == "bf16":
        return bf16_rne(y)
    raise ValueError(dtype)
