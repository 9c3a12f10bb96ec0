"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (no GPU needed: nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

import ternary_weight_quantized_bt_amd as bt
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "libternary.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bt_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("bt_pack_ternary", "bt_unpack_ternary", "bt_quant_act",
              "bt_quantize_weights", "bt_quantize_weights_workspace_bytes",
              "bt_dequantize_weights", "bt_i2s_import", "bt_i2s_export", "bt_i2s_bytes",
              "bt_b3_bytes", "bt_pack_ternary_b3", "bt_unpack_ternary_b3",
              "bt_ternary_gemv_b3",
              "bt_ternary_gemv", "bt_ternary_gemm", "bt_ternary_linear",
              "bt_linear_workspace_bytes", "bt_linear_one_launch", "bt_layer_forward",
              "bt_layer_workspace_bytes", "bt_layer_forward_noalloc",
              "bt_packed_bytes", "bt_last_error",
              "bt_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = bt.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert hasattr(bt, name), f"binding lacks {name}"


def test_abi_version():
    header = open(os.path.join(ROOT, "include", "libternary.h")).read()
    declared = int(re.search(r"#define BT_ABI_VERSION (\d+)", header).group(1))
    assert bt.bt_abi_version() == declared == bt.ABI_VERSION == 8


def test_packed_bytes():
    assert bt.bt_packed_bytes(2560, 2560) == 2560 * 2560 // 4 + 256
    assert bt.bt_packed_bytes(16, 256) == 16 * 256 // 4 + 256
    assert bt.bt_packed_bytes(15, 256) == 0
    assert "multiple of 16" in bt.bt_last_error()
    assert bt.bt_packed_bytes(16, 200) == 0
    assert bt.bt_packed_bytes(16, bt.BT_MAX_K + 256) == 0


A = 1 << 20  # a fake, 16-byte aligned address: never dereferenced because
             # validation fails before anything is launched


@pytest.mark.parametrize("args,status", [
    ((A, 15, 256, 1.0, A, None), bt.BT_ERR_SHAPE),
    ((A, 16, 300, 1.0, A, None), bt.BT_ERR_SHAPE),
    ((A, 0, 256, 1.0, A, None), bt.BT_ERR_SHAPE),
    ((None, 16, 256, 1.0, A, None), bt.BT_ERR_INVALID_ARG),
    ((A, 16, 256, 1.0, None, None), bt.BT_ERR_INVALID_ARG),
    ((A + 1, 16, 256, 1.0, A, None), bt.BT_ERR_ALIGN),
    ((A, 16, 256, 1.0, A, A + 2), bt.BT_ERR_ALIGN),
])
def test_pack_validation(args, status):
    with pytest.raises(bt.BtError) as e:
        bt.bt_pack_ternary(*args, stream=0)
    assert e.value.status == status


@pytest.mark.parametrize("fn", ["bt_ternary_gemv", "bt_ternary_gemm"])
@pytest.mark.parametrize("args,status", [
    ((A, 16, 256, A, A, A, -1, A, bt.BT_F32), bt.BT_ERR_INVALID_ARG),
    ((A, 16, 256, A, A, A, 1, A, 7), bt.BT_ERR_DTYPE),
    ((A, 16, 256 + 128, A, A, A, 1, A, bt.BT_F32), bt.BT_ERR_SHAPE),
    ((A, 16, bt.BT_MAX_K + 256, A, A, A, 1, A, bt.BT_F32), bt.BT_ERR_SHAPE),
    ((A, 16, 256, None, A, A, 1, A, bt.BT_F32), bt.BT_ERR_INVALID_ARG),
    ((A, 16, 256, A, None, A, 1, A, bt.BT_F32), bt.BT_ERR_INVALID_ARG),
    ((A, 16, 256, A, A, A, 1, A + 8, bt.BT_F32), bt.BT_ERR_ALIGN),
    ((A + 4, 16, 256, A, A, A, 1, A, bt.BT_F32), bt.BT_ERR_ALIGN),
])
def test_matmul_validation(fn, args, status):
    with pytest.raises(bt.BtError) as e:
        getattr(bt, fn)(*args, stream=0)
    assert e.value.status == status


def test_matmul_empty_batch_is_a_noop():
    # N = 0: validated, nothing launched, BT_OK (inputs may be NULL)
    bt.bt_ternary_gemv(A, 16, 256, None, None, None, 0, None, bt.BT_F32, stream=0)
    bt.bt_ternary_gemm(A, 16, 256, None, None, None, 0, None, bt.BT_BF16, stream=0)
    bt.bt_quant_act(None, bt.BT_BF16, 0, 256, None, None, None, stream=0)


@pytest.mark.parametrize("args,status", [
    ((A, bt.BT_I32, 1, 256, A, A, A), bt.BT_ERR_DTYPE),
    ((A, bt.BT_F32, 1, 100, A, A, A), bt.BT_ERR_SHAPE),
    ((A, bt.BT_F32, -3, 256, A, A, A), bt.BT_ERR_INVALID_ARG),
    ((A + 8, bt.BT_F32, 1, 256, A, A, A), bt.BT_ERR_ALIGN),
    ((A, bt.BT_F32, 1, 256, A, None, A), bt.BT_ERR_INVALID_ARG),
])
def test_quant_validation(args, status):
    with pytest.raises(bt.BtError) as e:
        bt.bt_quant_act(*args, stream=0)
    assert e.value.status == status


WQ = bt.BT_WQ_WORKSPACE_BYTES


@pytest.mark.parametrize("args,status", [
    ((A, bt.BT_F32, 15, 256, 0, 0.0, A, None, A, WQ), bt.BT_ERR_SHAPE),
    ((A, bt.BT_F32, 16, 200, 0, 0.0, A, None, A, WQ), bt.BT_ERR_SHAPE),
    ((A, bt.BT_F32, 1 << 24, 256, 0, 0.0, A, None, A, WQ), bt.BT_ERR_SHAPE),  # M*K > 2^31
    ((A, bt.BT_I32, 16, 256, 0, 0.0, A, None, A, WQ), bt.BT_ERR_DTYPE),
    ((A, bt.BT_F32, 16, 256, 2, 0.0, A, None, A, WQ), bt.BT_ERR_INVALID_ARG),
    ((A, bt.BT_F32, 16, 256, 0, -1e-5, A, None, A, WQ), bt.BT_ERR_INVALID_ARG),
    ((A, bt.BT_F32, 16, 256, 0, float("nan"), A, None, A, WQ), bt.BT_ERR_INVALID_ARG),
    ((A, bt.BT_F32, 16, 256, 0, float("inf"), A, None, A, WQ), bt.BT_ERR_INVALID_ARG),
    ((None, bt.BT_F32, 16, 256, 0, 0.0, A, None, A, WQ), bt.BT_ERR_INVALID_ARG),
    ((A, bt.BT_F32, 16, 256, 0, 0.0, None, None, A, WQ), bt.BT_ERR_INVALID_ARG),
    ((A + 4, bt.BT_F32, 16, 256, 0, 0.0, A, None, A, WQ), bt.BT_ERR_ALIGN),
    ((A, bt.BT_F32, 16, 256, 0, 0.0, A, A + 2, A, WQ), bt.BT_ERR_ALIGN),
    ((A, bt.BT_F32, 16, 256, 0, 0.0, A, None, None, WQ), bt.BT_ERR_WORKSPACE),
    ((A, bt.BT_F32, 16, 256, 0, 0.0, A, None, A, WQ - 1), bt.BT_ERR_WORKSPACE),
    ((A, bt.BT_F32, 16, 256, 0, 0.0, A, None, A + 8, WQ), bt.BT_ERR_ALIGN),
])
def test_quantize_weights_validation(args, status):
    with pytest.raises(bt.BtError) as e:
        bt.bt_quantize_weights(*args, stream=0)
    assert e.value.status == status


def test_quantize_weights_workspace_bytes():
    assert bt.bt_quantize_weights_workspace_bytes() == WQ == 4096


@pytest.mark.parametrize("fn,args,status", [
    ("bt_dequantize_weights", (A, 16, 256, A, bt.BT_I32), bt.BT_ERR_DTYPE),
    ("bt_dequantize_weights", (A, 15, 256, A, bt.BT_F32), bt.BT_ERR_SHAPE),
    ("bt_dequantize_weights", (None, 16, 256, A, bt.BT_F32), bt.BT_ERR_INVALID_ARG),
    ("bt_dequantize_weights", (A, 16, 256, A + 2, bt.BT_BF16), bt.BT_ERR_ALIGN),
    ("bt_i2s_import", (A, 16, 256, 6, A), bt.BT_ERR_SHAPE),
    ("bt_i2s_import", (A, 16, 256, 0, A), bt.BT_ERR_SHAPE),
    ("bt_i2s_import", (A, 16, 256, 3 * 256, A), bt.BT_ERR_SHAPE),  # does not divide M*K
    ("bt_i2s_import", (A, 16, 256, 128, None), bt.BT_ERR_INVALID_ARG),
    ("bt_i2s_import", (A + 1, 16, 256, 128, A), bt.BT_ERR_ALIGN),
    ("bt_i2s_export", (A, 16, 256, -4, A), bt.BT_ERR_SHAPE),
    ("bt_i2s_export", (A, 16, 200, 4, A), bt.BT_ERR_SHAPE),
    ("bt_i2s_export", (A, 16, 256, 4, None), bt.BT_ERR_INVALID_ARG),
])
def test_interop_validation(fn, args, status):
    with pytest.raises(bt.BtError) as e:
        getattr(bt, fn)(*args, stream=0)
    assert e.value.status == status


def test_b3_bytes():
    assert bt.bt_b3_bytes(16, 1024) == 16 * 1024 * 13 // 64 + 256
    assert bt.bt_b3_bytes(8192, 28672) == 8192 * 28672 * 13 // 64 + 256
    assert bt.bt_b3_bytes(16, 768) == 0
    assert "multiple of 1024" in bt.bt_last_error()
    assert bt.bt_b3_bytes(8, 1024) == 0
    assert bt.bt_b3_bytes(16, 132096) == 0  # above BT_MAX_K


@pytest.mark.parametrize("fn,args,status", [
    ("bt_pack_ternary_b3", (A, 16, 512, 1.0, A), bt.BT_ERR_SHAPE),
    ("bt_pack_ternary_b3", (A, 15, 1024, 1.0, A), bt.BT_ERR_SHAPE),
    ("bt_pack_ternary_b3", (None, 16, 1024, 1.0, A), bt.BT_ERR_INVALID_ARG),
    ("bt_pack_ternary_b3", (A, 16, 1024, 1.0, A + 4), bt.BT_ERR_ALIGN),
    ("bt_pack_ternary_b3", (A, 16, 1024, 1.0, A, A + 2), bt.BT_ERR_ALIGN),
    ("bt_unpack_ternary_b3", (A, 16, 2560, A), bt.BT_ERR_SHAPE),
    ("bt_unpack_ternary_b3", (A, 16, 1024, None), bt.BT_ERR_INVALID_ARG),
    ("bt_ternary_gemv_b3", (A, 16, 256, A, A, A, 1, A, bt.BT_F32), bt.BT_ERR_SHAPE),
    ("bt_ternary_gemv_b3", (A, 16, 1024, A, A, A, -1, A, bt.BT_F32), bt.BT_ERR_INVALID_ARG),
    ("bt_ternary_gemv_b3", (A, 16, 1024, A, A, A, 1, A, 7), bt.BT_ERR_DTYPE),
    ("bt_ternary_gemv_b3", (A, 16, 1024, None, A, A, 1, A, bt.BT_F32), bt.BT_ERR_INVALID_ARG),
    ("bt_ternary_gemv_b3", (A, 16, 1024, A, A, A, 1, A + 8, bt.BT_F32), bt.BT_ERR_ALIGN),
])
def test_b3_validation(fn, args, status):
    with pytest.raises(bt.BtError) as e:
        getattr(bt, fn)(*args, stream=0)
    assert e.value.status == status


def test_i2s_bytes():
    assert bt.bt_i2s_bytes(16, 256) == 16 * 256 // 4 + 4
    assert bt.bt_i2s_bytes(16, 100) == 0


def _layer(shapes):
    L = bt.bt_layer()
    for p, (M, K) in enumerate(shapes):
        L.w[p] = A
        L.M[p] = M
        L.K[p] = K
    return L


LAYER = [(64, 256), (32, 256), (32, 256), (256, 64 * 4), (96, 256), (96, 256),
         (256, 512)]


def test_layer_workspace_bytes():
    L = _layer(LAYER)
    n = bt.bt_layer_workspace_bytes(L, 5)
    # four inputs of widths 256, 256, 256, 512: int8 codes + scales + sums,
    # each block rounded up to 256 bytes
    expect = 0
    for K in (256, 256, 256, 512):
        expect += -(-5 * K // 256) * 256 + 256 + 256
    assert n == expect
    bad = list(LAYER)
    bad[1] = (32, 512)  # k and q must share K
    assert bt.bt_layer_workspace_bytes(_layer(bad), 5) == 0


def test_layer_validation():
    L = _layer(LAYER)
    io = bt.bt_layer_io()
    io.N = 3
    for i in range(4):
        io.x[i] = A
    for p in range(7):
        io.y[p] = A
    io.x_dtype = bt.BT_BF16
    io.y_dtype = bt.BT_BF16
    io.workspace = A
    io.workspace_bytes = 10
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_WORKSPACE
    io.workspace_bytes = 1 << 20
    io.x_dtype = bt.BT_I32
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_DTYPE
    io.x_dtype = bt.BT_F32
    io.y[6] = None
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_INVALID_ARG
    io.y[6] = A
    io.flags = 4  # not a defined flag
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_INVALID_ARG
    io.flags = bt.BT_LAYER_BASE3  # base-3 weights need K % 1024 == 0
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_SHAPE
    assert "1024" in bt.bt_last_error()
    io.flags = bt.BT_LAYER_PER_GROUP
    io.N = 0  # nothing to do
    bt.bt_layer_forward(L, io, stream=0)


def test_layer_one_launch_choice():
    """Host-side choice between the one-launch block kernel and per-group
    launches (no GPU work)."""
    big = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192),
           (28672, 8192), (8192, 28672)]
    small = [(2560, 2560), (640, 2560), (640, 2560), (2560, 2560), (6912, 2560),
             (6912, 2560), (2560, 6912)]
    assert bt.bt_layer_one_launch(_layer(big), 1, bt.BT_BF16) == 1
    assert bt.bt_layer_one_launch(_layer(big), 2, bt.BT_BF16) == 0   # chunks exceed registers
    assert bt.bt_layer_one_launch(_layer(big), 1, bt.BT_F32) == 0
    assert bt.bt_layer_one_launch(_layer(small), 3, bt.BT_BF16) == 1
    # 17.4 MB of packed weights: above the 12 MB up to which one launch beats
    # the matrix-core decode at 4 tokens
    assert bt.bt_layer_one_launch(_layer(small), 4, bt.BT_BF16) == 0
    assert bt.bt_layer_one_launch(_layer(small), 5, bt.BT_BF16) == 0
    # a 1B-class block (11.3 MB) still runs as one launch at 4 tokens; a
    # 13B-class one (79.3 MB) only at 1 token (64 MB limit at 2)
    tiny = [(2048, 2048), (512, 2048), (512, 2048), (2048, 2048), (5632, 2048),
            (5632, 2048), (2048, 5632)]
    assert bt.bt_layer_one_launch(_layer(tiny), 4, bt.BT_BF16) == 1
    b13 = [(5120, 5120)] * 4 + [(13824, 5120), (13824, 5120), (5120, 13824)]
    assert bt.bt_layer_one_launch(_layer(b13), 1, bt.BT_BF16) == 1
    assert bt.bt_layer_one_launch(_layer(b13), 2, bt.BT_BF16) == 0
    assert bt.bt_layer_one_launch(_layer(LAYER), 1, bt.BT_BF16) == 0  # K below 2048
    bad = list(LAYER)
    bad[1] = (32, 512)
    assert bt.bt_layer_one_launch(_layer(bad), 1, bt.BT_BF16) == -1


def test_linear_workspace_bytes():
    # codes [N, K], then scales and sums [N], each 256-byte aligned
    assert bt.bt_linear_workspace_bytes(8, 2560) == 20480 + 256 + 256
    assert bt.bt_linear_workspace_bytes(2048, 6912) == 2048 * 6912 + 8192 + 8192
    assert bt.bt_linear_workspace_bytes(3, 256) == 768 + 256 + 256
    assert bt.bt_linear_workspace_bytes(0, 256) == 0 + 0 + 0
    assert bt.bt_linear_workspace_bytes(-1, 256) == 0
    assert bt.bt_linear_workspace_bytes(1, 300) == 0


def test_linear_one_launch_choice():
    F, B = bt.BT_F32, bt.BT_BF16
    assert bt.bt_linear_one_launch(1, 2560, 2560, F) == 1
    assert bt.bt_linear_one_launch(1, 48, 32768, B) == 1    # 8 chunks per thread
    assert bt.bt_linear_one_launch(1, 48, 33024, B) == 0
    assert bt.bt_linear_one_launch(1, 48, 16384, F) == 1
    assert bt.bt_linear_one_launch(1, 48, 16640, F) == 0
    assert bt.bt_linear_one_launch(3, 208, 2304, B) == 1
    assert bt.bt_linear_one_launch(8, 4096, 2560, B) == 0   # matrix-core decode
    assert bt.bt_linear_one_launch(200, 64, 2560, B) == 0   # prefill
    assert bt.bt_linear_one_launch(0, 64, 2560, B) == 0
    assert bt.bt_linear_one_launch(1, 15, 2560, B) == -1
    assert bt.bt_linear_one_launch(1, 16, 2560, bt.BT_I32) == -1


@pytest.mark.parametrize("args,status", [
    ((A, 16, 256, A, bt.BT_I32, 1, A, bt.BT_F32, A, 1 << 20), bt.BT_ERR_DTYPE),
    ((A, 16, 256, A, bt.BT_F32, 1, A, 9, A, 1 << 20), bt.BT_ERR_DTYPE),
    ((A, 16, 300, A, bt.BT_F32, 1, A, bt.BT_F32, A, 1 << 20), bt.BT_ERR_SHAPE),
    ((A, 16, 256, A, bt.BT_F32, -2, A, bt.BT_F32, A, 1 << 20), bt.BT_ERR_INVALID_ARG),
    ((None, 16, 256, A, bt.BT_F32, 1, A, bt.BT_F32, A, 1 << 20), bt.BT_ERR_INVALID_ARG),
    ((A, 16, 256, None, bt.BT_F32, 1, A, bt.BT_F32, A, 1 << 20), bt.BT_ERR_INVALID_ARG),
    ((A, 16, 256, A + 4, bt.BT_F32, 1, A, bt.BT_F32, A, 1 << 20), bt.BT_ERR_ALIGN),
    ((A, 16, 256, A, bt.BT_F32, 1, A + 2, bt.BT_F32, A, 1 << 20), bt.BT_ERR_ALIGN),
    # through the workspace (8 tokens of a 4096-row matrix): missing, short,
    # misaligned -- all refused before anything is launched
    ((A, 4096, 2560, A, bt.BT_BF16, 8, A, bt.BT_F32, None, 0), bt.BT_ERR_WORKSPACE),
    ((A, 4096, 2560, A, bt.BT_BF16, 8, A, bt.BT_F32, A, 20991), bt.BT_ERR_WORKSPACE),
    ((A, 4096, 2560, A, bt.BT_BF16, 8, A, bt.BT_F32, A + 16, 1 << 20), bt.BT_ERR_ALIGN),
])
def test_linear_validation(args, status):
    with pytest.raises(bt.BtError) as e:
        bt.bt_ternary_linear(*args, stream=0)
    assert e.value.status == status


def test_linear_empty_batch_is_a_noop():
    bt.bt_ternary_linear(A, 16, 256, None, bt.BT_BF16, 0, None, bt.BT_F32, None, 0, stream=0)


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        bt.bt_ternary_gemv(torch.zeros(16), 16, 256, None, None, None, 0, None,
                           bt.BT_F32, stream=0)


def test_layer_noalloc_validation_on_the_host():
    """The allocation-free driver reports argument errors and scratch beyond
    its static array before it touches a device (nothing here launches)."""
    big = [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192), (28672, 8192),
           (28672, 8192), (8192, 28672)]
    L = _layer(big)
    io = bt.bt_layer_io()
    for i in range(4):
        io.x[i] = A
    for p in range(7):
        io.y[p] = A
    io.x_dtype = bt.BT_BF16
    io.y_dtype = bt.BT_I32
    # 640 tokens of this block need 34 MB of scratch: refused
    io.N = 640
    assert bt.bt_layer_workspace_bytes(L, 640) > bt.BT_NOALLOC_SCRATCH_BYTES
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward_noalloc(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_WORKSPACE
    assert "static scratch" in bt.bt_last_error()
    # other argument errors are the workspace driver's
    io.N = 8
    io.y_dtype = 9
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward_noalloc(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_DTYPE
    io.y_dtype = bt.BT_I32
    io.x[2] = None
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward_noalloc(L, io, stream=0)
    assert e.value.status == bt.BT_ERR_INVALID_ARG
    io.N = 0  # nothing to do, no device touched
    bt.bt_layer_forward_noalloc(L, io, stream=0)
    assert bt.BT_NOALLOC_SCRATCH_BYTES == 32 << 20
