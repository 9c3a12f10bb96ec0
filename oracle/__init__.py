"""CPU oracle for the ternary-weight x int8-activation product.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports this package and this package never imports the GPU library.

The arithmetic of the product path lives in ``bt_oracle.c`` (plain C, one
element at a time); this module only builds it with gcc and passes numpy
arrays through ctypes.  The readings of the pages it follows are listed in the
header of that file.  The float -> ternary weight quantizer (AbsMean and
max|w| scales, RoundClip) is ``weight_quant.py``: numpy plus exact Python
integer arithmetic, its readings in its own header.  Dequantization
(to_float) and the I2_S byte layout are ``interop.py`` (numpy).  The denser
base-3 packing (64 weights in 13 bytes) is ``base3.py`` (numpy).

Sources, cited by page title and section:
  [I2S]  "How BitNet's 1-Bit (I2_S) Quantization Works Compared to Standard
         LLM Quantization" -- "Ternary Representation and Packing",
         "Per-Tensor Scaling Strategy", "How I2_S Kernels Process the Format".
  [PARA] "LLM Quantization Paradigms: FP8, AWQ, EXL2 & BitNet b1.58 in 2026"
         -- section 5 (figure "BitNet b1.58 Ternary Matrix Multiplication",
         the AbsMean / RoundClip equations and Quant8).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bt_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fopenmp", "-shared", "-fPIC"]
# A checking build of the same source (host code only): address and
# undefined-behaviour sanitizers, float-to-int conversions out of range
# included, every report fatal.  Loading it needs the address sanitizer's
# runtime preloaded into the process.
SANITIZE_FLAGS = ["-g", "-fno-omit-frame-pointer",
                  "-fsanitize=address,undefined,float-cast-overflow",
                  "-fno-sanitize-recover=all"]
# Set to the path of another build of bt_oracle.c (e.g. the checking build)
# to load that one instead.
LIB_ENV = "BT_ORACLE_SO"

_lib = None


def build(force: bool = True) -> str:
    """Compile bt_oracle.c into liboracle.so next to it (gcc)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile bt_oracle.c with SANITIZE_FLAGS into `path`."""
    subprocess.run(["gcc", *CFLAGS, *SANITIZE_FLAGS, "-o", path, _SRC, "-lm"], check=True)
    return path


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get(LIB_ENV)
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or (
                    os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.bto_packed_bytes.argtypes = [I, I]
        lib.bto_packed_bytes.restype = I
        lib.bto_pack.argtypes = [P, I, I, ctypes.c_float, P]
        lib.bto_pack.restype = I
        lib.bto_unpack.argtypes = [P, I, I, P]
        lib.bto_unpack.restype = None
        lib.bto_scale.argtypes = [P, I, I]
        lib.bto_scale.restype = ctypes.c_float
        lib.bto_quant_act_f32.argtypes = [P, I, I, P, P, P]
        lib.bto_quant_act_f32.restype = None
        lib.bto_quant_act_bf16.argtypes = [P, I, I, P, P, P]
        lib.bto_quant_act_bf16.restype = None
        lib.bto_matmul_i32.argtypes = [P, I, I, P, I, P, I, P]
        lib.bto_matmul_i32.restype = ctypes.c_int
        lib.bto_dequant.argtypes = [P, I, I, ctypes.c_double, P, P]
        lib.bto_dequant.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _check_shape(M: int, K: int):
    if M % 16 or K % 256:
        raise ValueError(f"oracle layout needs M%16==0 and K%256==0 (M={M}, K={K})")


def packed_bytes(M: int, K: int) -> int:
    return int(_load().bto_packed_bytes(M, K))


def pack(w: np.ndarray, scale: float):
    """int8 w[M,K] -> (packed uint8 buffer, count of values outside {-1,0,1})."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    M, K = w.shape
    _check_shape(M, K)
    out = np.empty(packed_bytes(M, K), dtype=np.uint8)
    bad = _load().bto_pack(_ptr(w), M, K, ctypes.c_float(scale), _ptr(out))
    return out, int(bad)


def unpack(packed: np.ndarray, M: int, K: int) -> np.ndarray:
    _check_shape(M, K)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size >= packed_bytes(M, K)
    w = np.empty((M, K), dtype=np.int8)
    _load().bto_unpack(_ptr(packed), M, K, _ptr(w))
    return w


def scale_of(packed: np.ndarray, M: int, K: int) -> float:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    return float(_load().bto_scale(_ptr(packed), M, K))


def quant_act(x: np.ndarray):
    """Per-token absmax int8 quantization.

    x is float32 [N,K] or bfloat16 bits as uint16 [N,K].
    Returns (xq int8 [N,K], scale float32 [N], sum int32 [N]).
    """
    x = np.ascontiguousarray(x)
    N, K = x.shape
    xq = np.empty((N, K), dtype=np.int8)
    s = np.empty(N, dtype=np.float32)
    sm = np.empty(N, dtype=np.int32)
    if x.dtype == np.float32:
        _load().bto_quant_act_f32(_ptr(x), N, K, _ptr(xq), _ptr(s), _ptr(sm))
    elif x.dtype == np.uint16:
        _load().bto_quant_act_bf16(_ptr(x), N, K, _ptr(xq), _ptr(s), _ptr(sm))
    else:
        raise TypeError("x must be float32 or bfloat16 bits (uint16)")
    return xq, s, sm


def matmul_i32(packed: np.ndarray, M: int, K: int, xq: np.ndarray,
               rows: np.ndarray | None = None) -> np.ndarray:
    """acc[n, j] = sum_k W[rows[j], k] * xq[n, k]  (all rows if rows is None)."""
    _check_shape(M, K)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    N = xq.shape[0]
    assert xq.shape[1] == K
    if rows is None:
        nrows, rp = M, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.min(initial=0) >= 0 and rows.max(initial=0) < M
        nrows, rp = rows.size, _ptr(rows)
    acc = np.empty((N, nrows), dtype=np.int32)
    if N and nrows:
        bad = _load().bto_matmul_i32(_ptr(packed), M, K, rp, nrows, _ptr(xq),
                                     N, _ptr(acc))
        if bad:
            raise OverflowError("ternary dot product does not fit int32")
    return acc


def dequant(acc: np.ndarray, s_w: float, s_a: np.ndarray) -> np.ndarray:
    """y = acc * s_w * s_a[n] / 127 in float64."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s_a = np.ascontiguousarray(s_a, dtype=np.float32)
    N, C = acc.shape
    y = np.empty((N, C), dtype=np.float64)
    _load().bto_dequant(_ptr(acc), N, C, ctypes.c_double(s_w), _ptr(s_a), _ptr(y))
    return y


def forward(packed: np.ndarray, M: int, K: int, x: np.ndarray,
            rows: np.ndarray | None = None):
    """Whole path for one projection: quantize x, integer product, dequantize.

    Returns dict with xq, x_scale, x_sum, acc and y (float64)."""
    xq, s, sm = quant_act(x)
    acc = matmul_i32(packed, M, K, xq, rows)
    y = dequant(acc, scale_of(packed, M, K), s)
    return {"xq": xq, "x_scale": s, "x_sum": sm, "acc": acc, "y": y}
