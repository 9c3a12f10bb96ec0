"""Python binding of libternary (ternary-weight x int8-activation product on
AMD MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libternary.so``.  PyTorch supplies device memory and the current
stream.  The functions named ``bt_*`` mirror the C ABI in
``include/libternary.h`` one to one (same names, same argument order; tensors
are passed as device pointers).  A few helpers below (``pack``,
``quant_act``, ``gemv``, ``gemm``, ``Layer``) allocate the outputs with
``torch.empty`` and call them.

If ``libternary.so`` has not been built, importing the binding succeeds but
every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libternary.so")

BT_OK = 0
BT_ERR_INVALID_ARG = 1
BT_ERR_SHAPE = 2
BT_ERR_ALIGN = 3
BT_ERR_DTYPE = 4
BT_ERR_HIP = 5
BT_ERR_WORKSPACE = 6
STATUS_NAMES = {0: "BT_OK", 1: "BT_ERR_INVALID_ARG", 2: "BT_ERR_SHAPE",
                3: "BT_ERR_ALIGN", 4: "BT_ERR_DTYPE", 5: "BT_ERR_HIP",
                6: "BT_ERR_WORKSPACE"}

BT_F32 = 0
BT_BF16 = 1
BT_I32 = 2
BT_MAX_K = 131840
BT_MAX_N = 2097152  # tokens per call
BT_LAYER_PROJ = 7
BT_LAYER_INPUTS = 4

_TORCH_DTYPE = {BT_F32: torch.float32, BT_BF16: torch.bfloat16, BT_I32: torch.int32}
_BT_DTYPE = {torch.float32: BT_F32, torch.bfloat16: BT_BF16, torch.int32: BT_I32}


class BtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


BT_MAX_GROUP = 3
BT_PREFILL_MIN_N = 128


class bt_proj(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p),
                ("M", ctypes.c_int64),
                ("y", ctypes.c_void_p)]


class bt_layer(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p * BT_LAYER_PROJ),
                ("M", ctypes.c_int64 * BT_LAYER_PROJ),
                ("K", ctypes.c_int64 * BT_LAYER_PROJ)]


class bt_layer_io(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64),
                ("x", ctypes.c_void_p * BT_LAYER_INPUTS),
                ("x_dtype", ctypes.c_int),
                ("y", ctypes.c_void_p * BT_LAYER_PROJ),
                ("y_dtype", ctypes.c_int),
                ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t),
                ("flags", ctypes.c_uint32)]


BT_LAYER_PER_GROUP = 1
BT_LAYER_BASE3 = 2
BT_WSCALE_ABSMEAN = 0
BT_WSCALE_ABSMAX = 1
BT_WQ_WORKSPACE_BYTES = 4096

# The C ABI version these structures and signatures follow (BT_ABI_VERSION).
ABI_VERSION = 8

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libternary.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m ternary_weight_quantized_bt_amd.build` "
                "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.bt_abi_version.argtypes = []
        L.bt_abi_version.restype = ctypes.c_int
        if L.bt_abi_version() != ABI_VERSION:
            raise RuntimeError(
                f"{LIB_PATH} has C ABI version {L.bt_abi_version()}, this binding "
                f"expects {ABI_VERSION}: rebuild it")
        L.bt_last_error.argtypes = []
        L.bt_last_error.restype = ctypes.c_char_p
        L.bt_packed_bytes.argtypes = [I64, I64]
        L.bt_packed_bytes.restype = ctypes.c_size_t
        L.bt_pack_ternary.argtypes = [P, I64, I64, ctypes.c_float, P, P, P]
        L.bt_pack_ternary.restype = S
        L.bt_unpack_ternary.argtypes = [P, I64, I64, P, P]
        L.bt_unpack_ternary.restype = S
        L.bt_i2s_bytes.argtypes = [I64, I64]
        L.bt_i2s_bytes.restype = ctypes.c_size_t
        L.bt_dequantize_weights.argtypes = [P, I64, I64, P, S, P]
        L.bt_dequantize_weights.restype = S
        L.bt_i2s_import.argtypes = [P, I64, I64, I64, P, P, P]
        L.bt_i2s_import.restype = S
        L.bt_i2s_export.argtypes = [P, I64, I64, I64, P, P]
        L.bt_i2s_export.restype = S
        L.bt_b3_bytes.argtypes = [I64, I64]
        L.bt_b3_bytes.restype = ctypes.c_size_t
        L.bt_pack_ternary_b3.argtypes = [P, I64, I64, ctypes.c_float, P, P, P]
        L.bt_pack_ternary_b3.restype = S
        L.bt_unpack_ternary_b3.argtypes = [P, I64, I64, P, P]
        L.bt_unpack_ternary_b3.restype = S
        L.bt_ternary_gemv_b3.argtypes = [P, I64, I64, P, P, P, I64, P, S, P]
        L.bt_ternary_gemv_b3.restype = S
        L.bt_quantize_weights_workspace_bytes.argtypes = []
        L.bt_quantize_weights_workspace_bytes.restype = ctypes.c_size_t
        L.bt_quantize_weights.argtypes = [P, S, I64, I64, S, ctypes.c_float, P, P, P,
                                          ctypes.c_size_t, P]
        L.bt_quantize_weights.restype = S
        L.bt_quant_act.argtypes = [P, S, I64, I64, P, P, P, P]
        L.bt_quant_act.restype = S
        for fn in (L.bt_ternary_gemv, L.bt_ternary_gemm):
            fn.argtypes = [P, I64, I64, P, P, P, I64, P, S, P]
            fn.restype = S
        L.bt_ternary_matmul_group.argtypes = [ctypes.POINTER(bt_proj), S, I64, P, P,
                                              P, I64, S, P]
        L.bt_ternary_matmul_group.restype = S
        L.bt_linear_workspace_bytes.argtypes = [I64, I64]
        L.bt_linear_workspace_bytes.restype = ctypes.c_size_t
        L.bt_linear_one_launch.argtypes = [I64, I64, I64, S]
        L.bt_linear_one_launch.restype = S
        L.bt_ternary_linear.argtypes = [P, I64, I64, P, S, I64, P, S, P, ctypes.c_size_t, P]
        L.bt_ternary_linear.restype = S
        L.bt_layer_one_launch.argtypes = [ctypes.POINTER(bt_layer), I64, S]
        L.bt_layer_one_launch.restype = S
        L.bt_layer_workspace_bytes.argtypes = [ctypes.POINTER(bt_layer), I64]
        L.bt_layer_workspace_bytes.restype = ctypes.c_size_t
        L.bt_layer_forward.argtypes = [ctypes.POINTER(bt_layer),
                                       ctypes.POINTER(bt_layer_io), P]
        L.bt_layer_forward.restype = S
        L.bt_layer_forward_noalloc.argtypes = [ctypes.POINTER(bt_layer),
                                               ctypes.POINTER(bt_layer_io), P]
        L.bt_layer_forward_noalloc.restype = S
        _lib = L
    return _lib


def _p(t):
    """Device pointer of a tensor (or None / a raw integer address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a tensor, got {type(t)}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if t.numel() and not t.is_cuda:
        raise ValueError("tensor must live in GPU memory")
    return t.data_ptr() if t.numel() else None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int):
    if status != BT_OK:
        raise BtError(status, lib().bt_last_error().decode())


def _keep_for_stream(tensors, stream):
    """Tensors allocated here on the current stream but used by kernels on
    another stream: tell torch's caching allocator, so their memory is not
    handed out again before that stream's work is done."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if t is not None and t.numel():
            t.record_stream(s)


def _out(out, shape, dtype, device, what):
    """A caller-supplied output tensor (checked), or a new one."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype:
        raise ValueError(f"{what}: expected {tuple(shape)} {dtype}, got "
                         f"{tuple(out.shape)} {out.dtype}")
    return out


# ---------------------------------------------------------------- C ABI ----

def bt_abi_version() -> int:
    return lib().bt_abi_version()


def bt_last_error() -> str:
    return lib().bt_last_error().decode()


def bt_packed_bytes(M: int, K: int) -> int:
    return lib().bt_packed_bytes(M, K)


def bt_pack_ternary(w, M, K, scale, packed, invalid_count=None, stream=None):
    _check(lib().bt_pack_ternary(_p(w), M, K, float(scale), _p(packed),
                                 _p(invalid_count), _stream(stream)))


def bt_unpack_ternary(packed, M, K, w, stream=None):
    _check(lib().bt_unpack_ternary(_p(packed), M, K, _p(w), _stream(stream)))


def bt_i2s_bytes(M: int, K: int) -> int:
    return lib().bt_i2s_bytes(M, K)


def bt_dequantize_weights(packed, M, K, w, w_dtype, stream=None):
    _check(lib().bt_dequantize_weights(_p(packed), M, K, _p(w), w_dtype, _stream(stream)))


def bt_i2s_import(i2s, M, K, block, packed, invalid_count=None, stream=None):
    _check(lib().bt_i2s_import(_p(i2s), M, K, block, _p(packed), _p(invalid_count),
                               _stream(stream)))


def bt_i2s_export(packed, M, K, block, i2s, stream=None):
    _check(lib().bt_i2s_export(_p(packed), M, K, block, _p(i2s), _stream(stream)))


def bt_b3_bytes(M: int, K: int) -> int:
    return lib().bt_b3_bytes(M, K)


def bt_pack_ternary_b3(w, M, K, scale, packed, invalid_count=None, stream=None):
    _check(lib().bt_pack_ternary_b3(_p(w), M, K, float(scale), _p(packed),
                                    _p(invalid_count), _stream(stream)))


def bt_unpack_ternary_b3(packed, M, K, w, stream=None):
    _check(lib().bt_unpack_ternary_b3(_p(packed), M, K, _p(w), _stream(stream)))


def bt_ternary_gemv_b3(packed, M, K, xq, x_scale, x_sum, N, y, y_dtype, stream=None):
    _check(lib().bt_ternary_gemv_b3(_p(packed), M, K, _p(xq), _p(x_scale), _p(x_sum),
                                    N, _p(y), y_dtype, _stream(stream)))


def bt_quantize_weights_workspace_bytes() -> int:
    return lib().bt_quantize_weights_workspace_bytes()


def bt_quantize_weights(w, w_dtype, M, K, scale_mode, eps, packed, stats, workspace,
                        workspace_bytes, stream=None):
    _check(lib().bt_quantize_weights(_p(w), w_dtype, M, K, scale_mode, float(eps),
                                     _p(packed), _p(stats), _p(workspace),
                                     workspace_bytes, _stream(stream)))


def bt_quant_act(x, x_dtype, N, K, xq, x_scale, x_sum, stream=None):
    _check(lib().bt_quant_act(_p(x), x_dtype, N, K, _p(xq), _p(x_scale),
                              _p(x_sum), _stream(stream)))


def bt_ternary_gemv(packed, M, K, xq, x_scale, x_sum, N, y, y_dtype, stream=None):
    _check(lib().bt_ternary_gemv(_p(packed), M, K, _p(xq), _p(x_scale), _p(x_sum),
                                 N, _p(y), y_dtype, _stream(stream)))


def bt_ternary_gemm(packed, M, K, xq, x_scale, x_sum, N, y, y_dtype, stream=None):
    _check(lib().bt_ternary_gemm(_p(packed), M, K, _p(xq), _p(x_scale), _p(x_sum),
                                 N, _p(y), y_dtype, _stream(stream)))


def bt_ternary_matmul_group(projs, count, K, xq, x_scale, x_sum, N, y_dtype,
                            stream=None):
    """projs: a ctypes array of bt_proj (see make_projs)."""
    _check(lib().bt_ternary_matmul_group(projs, count, K, _p(xq), _p(x_scale),
                                         _p(x_sum), N, y_dtype, _stream(stream)))


def bt_linear_workspace_bytes(N: int, K: int) -> int:
    return lib().bt_linear_workspace_bytes(N, K)


def bt_linear_one_launch(N: int, M: int, K: int, x_dtype: int) -> int:
    return lib().bt_linear_one_launch(N, M, K, x_dtype)


def bt_ternary_linear(packed, M, K, x, x_dtype, N, y, y_dtype, workspace,
                      workspace_bytes, stream=None):
    _check(lib().bt_ternary_linear(_p(packed), M, K, _p(x), x_dtype, N, _p(y), y_dtype,
                                   _p(workspace), workspace_bytes, _stream(stream)))


def make_projs(items):
    """[(packed tensor, M, y tensor), ...] -> ctypes array of bt_proj."""
    arr = (bt_proj * len(items))()
    for i, (packed, M, y) in enumerate(items):
        arr[i].packed = _p(packed)
        arr[i].M = M
        arr[i].y = _p(y)
    return arr


def bt_layer_one_launch(layer: bt_layer, N: int, x_dtype: int) -> int:
    return lib().bt_layer_one_launch(ctypes.byref(layer), N, x_dtype)


def bt_layer_workspace_bytes(layer: bt_layer, N: int) -> int:
    return lib().bt_layer_workspace_bytes(ctypes.byref(layer), N)


def bt_layer_forward(layer: bt_layer, io: bt_layer_io, stream=None):
    _check(lib().bt_layer_forward(ctypes.byref(layer), ctypes.byref(io),
                                  _stream(stream)))


BT_NOALLOC_SCRATCH_BYTES = 32 << 20


def bt_layer_forward_noalloc(layer: bt_layer, io: bt_layer_io, stream=None):
    _check(lib().bt_layer_forward_noalloc(ctypes.byref(layer), ctypes.byref(io),
                                          _stream(stream)))


# -------------------------------------------------------------- helpers ----

def _check_packed(packed, n, what):
    if packed.dtype != torch.uint8 or packed.numel() != n:
        raise ValueError(f"{what}: packed weights must be {n} uint8 bytes, got "
                         f"{packed.numel()} {packed.dtype}")


def pack(w: torch.Tensor, scale: float, invalid_count=None, stream=None, out=None):
    """int8 [M, K] device tensor -> packed uint8 device tensor."""
    M, K = w.shape
    n = bt_packed_bytes(M, K)
    if n == 0:
        raise BtError(BT_ERR_SHAPE, bt_last_error())
    packed = _out(out, (n,), torch.uint8, w.device, "pack")
    bt_pack_ternary(w, M, K, scale, packed, invalid_count, stream)
    return packed


def unpack(packed: torch.Tensor, M: int, K: int, stream=None, out=None):
    w = _out(out, (M, K), torch.int8, packed.device, "unpack")
    bt_unpack_ternary(packed, M, K, w, stream)
    return w


def pack_b3(w: torch.Tensor, scale: float, invalid_count=None, stream=None, out=None):
    """int8 [M, K] device tensor -> base-3 B3T1024 packed uint8 device tensor."""
    M, K = w.shape
    n = bt_b3_bytes(M, K)
    if n == 0:
        raise BtError(BT_ERR_SHAPE, bt_last_error())
    packed = _out(out, (n,), torch.uint8, w.device, "pack_b3")
    bt_pack_ternary_b3(w, M, K, scale, packed, invalid_count, stream)
    return packed


def unpack_b3(packed: torch.Tensor, M: int, K: int, stream=None, out=None):
    w = _out(out, (M, K), torch.int8, packed.device, "unpack_b3")
    bt_unpack_ternary_b3(packed, M, K, w, stream)
    return w


def dequantize(packed: torch.Tensor, M: int, K: int, dtype=torch.float32, stream=None,
               out=None):
    """Packed weights -> float32 / bfloat16 [M, K] device tensor
    ((code - 1) * scale)."""
    w = _out(out, (M, K), dtype, packed.device, "dequantize")
    bt_dequantize_weights(packed, M, K, w, _BT_DTYPE[dtype], stream)
    return w


def i2s_import(i2s: torch.Tensor, M: int, K: int, block: int, invalid_count=None,
               stream=None, out=None):
    """I2_S bytes (blocks of `block` weights) -> packed T16Q256 tensor."""
    n = bt_packed_bytes(M, K)
    if n == 0:
        raise BtError(BT_ERR_SHAPE, bt_last_error())
    packed = _out(out, (n,), torch.uint8, i2s.device, "i2s_import")
    bt_i2s_import(i2s, M, K, block, packed, invalid_count, stream)
    return packed


def i2s_export(packed: torch.Tensor, M: int, K: int, block: int, stream=None, out=None):
    """Packed T16Q256 tensor -> I2_S bytes (blocks of `block` weights)."""
    n = bt_i2s_bytes(M, K)
    if n == 0:
        raise BtError(BT_ERR_SHAPE, bt_last_error())
    res = _out(out, (n,), torch.uint8, packed.device, "i2s_export")
    bt_i2s_export(packed, M, K, block, res, stream)
    return res


def quantize_weights(w: torch.Tensor, mode: str = "absmean", eps: float = 0.0,
                     stream=None):
    """float32 / bfloat16 [M, K] device weights -> (packed uint8 tensor with
    the scale d in its tail, stats float32 [2] = (s, d)); mode "absmean"
    (s = mean |W|) or "absmax" (s = max |W|), d = s + eps."""
    M, K = w.shape
    n = bt_packed_bytes(M, K)
    if n == 0:
        raise BtError(BT_ERR_SHAPE, bt_last_error())
    modes = {"absmean": BT_WSCALE_ABSMEAN, "absmax": BT_WSCALE_ABSMAX}
    if mode not in modes:
        raise ValueError(f"mode must be one of {sorted(modes)}")
    dev = w.device
    packed = torch.empty(n, dtype=torch.uint8, device=dev)
    stats = torch.empty(2, dtype=torch.float32, device=dev)
    ws_bytes = bt_quantize_weights_workspace_bytes()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    bt_quantize_weights(w, _BT_DTYPE[w.dtype], M, K, modes[mode], eps, packed, stats,
                        ws, ws_bytes, stream)
    _keep_for_stream((ws, packed, stats), stream)
    return packed, stats


def quant_act(x: torch.Tensor, stream=None, out=None):
    """float32 / bfloat16 [N, K] -> (xq int8 [N, K], scale f32 [N], sum i32 [N]);
    out, if given, is such a triple to write into."""
    N, K = x.shape
    dev = x.device
    o = out if out is not None else (None, None, None)
    xq = _out(o[0], (N, K), torch.int8, dev, "quant_act xq")
    s = _out(o[1], (N,), torch.float32, dev, "quant_act scale")
    sm = _out(o[2], (N,), torch.int32, dev, "quant_act sum")
    bt_quant_act(x, _BT_DTYPE[x.dtype], N, K, xq, s, sm, stream)
    return xq, s, sm


def _matmul(fn, packed, M, K, xq, xs, xsum, y_dtype, stream, y, b3=False):
    N = xq.shape[0]
    if tuple(xq.shape) != (N, K) or xq.dtype != torch.int8:
        raise ValueError(f"xq must be int8 [N, {K}], got {tuple(xq.shape)} {xq.dtype}")
    if tuple(xs.shape) != (N,) or tuple(xsum.shape) != (N,):
        raise ValueError("x_scale and x_sum must have one entry per token")
    _check_packed(packed, bt_b3_bytes(M, K) if b3 else bt_packed_bytes(M, K), "matmul")
    y = _out(y, (N, M), _TORCH_DTYPE[y_dtype], xq.device, "matmul y")
    fn(packed, M, K, xq, xs, xsum, N, y, y_dtype, stream)
    return y


def gemv(packed, M, K, xq, xs, xsum, y_dtype=BT_F32, stream=None, y=None):
    return _matmul(bt_ternary_gemv, packed, M, K, xq, xs, xsum, y_dtype, stream, y)


def gemv_b3(packed, M, K, xq, xs, xsum, y_dtype=BT_F32, stream=None, y=None):
    """The decode product over base-3 B3T1024 weights (same results as gemv)."""
    return _matmul(bt_ternary_gemv_b3, packed, M, K, xq, xs, xsum, y_dtype, stream, y,
                   b3=True)


def gemm(packed, M, K, xq, xs, xsum, y_dtype=BT_F32, stream=None, y=None):
    return _matmul(bt_ternary_gemm, packed, M, K, xq, xs, xsum, y_dtype, stream, y)


def linear(packed, M, K, x, y_dtype=BT_F32, workspace=None, stream=None, y=None):
    """float32 / bfloat16 x [N, K] -> y [N, M]: quantization and product in
    one call (one launch where the decode kernel quantizes the tokens itself,
    else through a workspace, allocated here unless given)."""
    N = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K or x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"x must be float32 / bfloat16 [N, {K}], got "
                         f"{tuple(x.shape)} {x.dtype}")
    _check_packed(packed, bt_packed_bytes(M, K), "linear")
    y = _out(y, (N, M), _TORCH_DTYPE[y_dtype], x.device, "linear y")
    xdt = _BT_DTYPE[x.dtype]
    need = 0 if bt_linear_one_launch(N, M, K, xdt) == 1 else bt_linear_workspace_bytes(N, K)
    made = None
    if workspace is None and need:
        made = workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wbytes = workspace.numel() if workspace is not None else 0
    bt_ternary_linear(packed, M, K, x, xdt, N, y, y_dtype, workspace, wbytes, stream)
    _keep_for_stream((made,), stream)
    return y


class Layer:
    """Seven packed projections (q, k, v, o, gate, up, down) of one block
    (T16Q256 bytes, or base-3 B3T1024 bytes with base3=True)."""

    def __init__(self, packed, shapes, base3=False):
        assert len(packed) == BT_LAYER_PROJ and len(shapes) == BT_LAYER_PROJ
        self.packed = list(packed)  # keeps the tensors alive
        self.shapes = [tuple(s) for s in shapes]
        self.base3 = base3
        self.c = bt_layer()
        for p, (t, (M, K)) in enumerate(zip(self.packed, self.shapes)):
            _check_packed(t, bt_b3_bytes(M, K) if base3 else bt_packed_bytes(M, K),
                          f"layer projection {p}")
            self.c.w[p] = _p(t)
            self.c.M[p] = M
            self.c.K[p] = K

    def workspace_bytes(self, N: int) -> int:
        return bt_layer_workspace_bytes(self.c, N)

    def make_io(self, xs, ys, y_dtype, workspace, per_group=False) -> bt_layer_io:
        io = bt_layer_io()
        io.flags = (BT_LAYER_PER_GROUP if per_group else 0) | (BT_LAYER_BASE3 if self.base3 else 0)
        io.N = xs[0].shape[0]
        for i, x in enumerate(xs):
            io.x[i] = _p(x)
        io.x_dtype = _BT_DTYPE[xs[0].dtype]
        for p, y in enumerate(ys):
            io.y[p] = _p(y)
        io.y_dtype = y_dtype
        io.workspace = _p(workspace)
        io.workspace_bytes = workspace.numel() if workspace is not None else 0
        return io

    def alloc_outputs(self, N: int, y_dtype: int, device):
        return [torch.empty((N, M), dtype=_TORCH_DTYPE[y_dtype], device=device)
                for (M, _) in self.shapes]

    def alloc_workspace(self, N: int, device):
        # 256-byte alignment: torch's caching allocator returns at least
        # 512-byte aligned blocks.
        return torch.empty(max(self.workspace_bytes(N), 256), dtype=torch.uint8,
                           device=device)

    def input_widths(self):
        """K of the four inputs (q/k/v, o, gate/up, down)."""
        return [self.shapes[0][1], self.shapes[3][1], self.shapes[4][1], self.shapes[6][1]]

    def check_io(self, xs, ys, y_dtype):
        """Shapes, dtypes and devices of the inputs and outputs: a mismatch
        would make the kernels read or write out of bounds."""
        if len(xs) != BT_LAYER_INPUTS:
            raise ValueError(f"need {BT_LAYER_INPUTS} inputs, got {len(xs)}")
        N, dt = xs[0].shape[0], xs[0].dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise ValueError(f"inputs must be float32 or bfloat16, got {dt}")
        for i, (x, K) in enumerate(zip(xs, self.input_widths())):
            if x.dim() != 2 or tuple(x.shape) != (N, K) or x.dtype != dt or not x.is_cuda:
                raise ValueError(f"input {i}: expected a GPU tensor [{N}, {K}] {dt}, got "
                                 f"{tuple(x.shape)} {x.dtype} on {x.device}")
        if len(ys) != BT_LAYER_PROJ:
            raise ValueError(f"need {BT_LAYER_PROJ} outputs, got {len(ys)}")
        for p, (y, (M, _)) in enumerate(zip(ys, self.shapes)):
            if tuple(y.shape) != (N, M) or y.dtype != _TORCH_DTYPE[y_dtype] or not y.is_cuda:
                raise ValueError(f"output {p}: expected a GPU tensor [{N}, {M}] "
                                 f"{_TORCH_DTYPE[y_dtype]}, got {tuple(y.shape)} {y.dtype}")

    def forward(self, xs, y_dtype=BT_BF16, ys=None, workspace=None, stream=None,
                per_group=False):
        N = xs[0].shape[0]
        dev = xs[0].device
        own_ws, own_ys = workspace is None, ys is None
        if own_ys:
            ys = self.alloc_outputs(N, y_dtype, dev)
        self.check_io(xs, ys, y_dtype)
        if own_ws:
            workspace = self.alloc_workspace(N, dev)
        io = self.make_io(xs, ys, y_dtype, workspace, per_group)
        bt_layer_forward(self.c, io, stream)
        _keep_for_stream(([workspace] if own_ws else []) + (list(ys) if own_ys else []), stream)
        return ys
