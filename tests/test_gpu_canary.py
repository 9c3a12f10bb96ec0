"""Sentinel bands around every output, one test per kernel path: a kernel that
writes past either end of its output changes a band byte.  Each case also
checks its results against the oracle, so a kernel that writes inside the
buffer but in the wrong place fails too.

Paths: pack and unpack (2-bit and base-3), activation quantization, the
single-token decode kernel (dot4, 1..4 tokens, with and without the fused
quantization), the matrix-core decode (5..127 tokens, one and several K
phases), the prefill kernel (the whole-row bf16 store path and the per-lane
path), the one-launch block kernel, the base-3 decode, and the weight
dequantization and I2_S conversions."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt
import workloads as W
from oracle import base3, interop
from parity import Guarded, assert_equal, check_projection, to_np, x_for_oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
TORCH_DT = {bt.BT_I32: torch.int32, bt.BT_F32: torch.float32, bt.BT_BF16: torch.bfloat16}


def _weights(M, K, seed):
    return W.ternary_weights(M, K, "p0_0.4", seed)


def test_pack_unpack_and_quant():
    M, K, N = 80, 768, 5
    w = _weights(M, K, 11)
    gp = Guarded((bt.bt_packed_bytes(M, K),), torch.uint8)
    bt.pack(w.to(DEV), 0.03, out=gp.t)
    gu = Guarded((M, K), torch.int8)
    bt.unpack(gp.t, M, K, out=gu.t)
    x = W.activations(N, K, "normal", 12, "bf16", 0.01, 20.0)
    gq = [Guarded((N, K), torch.int8), Guarded((N,), torch.float32), Guarded((N,), torch.int32)]
    bt.quant_act(x.to(DEV), out=tuple(g.t for g in gq))
    torch.cuda.synchronize()
    for g, what in [(gp, "pack"), (gu, "unpack"), (gq[0], "xq"), (gq[1], "scale"),
                    (gq[2], "sum")]:
        g.check(what)
    ref, _ = oracle.pack(w.numpy(), 0.03)
    assert_equal(to_np(gp.t), ref, "packed")
    assert_equal(to_np(gu.t), w.numpy(), "unpacked")
    xq, xs, xsum = oracle.quant_act(x_for_oracle(x))
    assert_equal(to_np(gq[0].t), xq, "xq")
    assert_equal(to_np(gq[1].t), xs, "scale")
    assert_equal(to_np(gq[2].t), xsum, "sum")


# 1..4 tokens: dot4 decode; 5, 17, 64, 127: matrix-core decode (K = 9216 at
# 64 and 127 tokens needs two K phases); 128, 200: prefill.
@pytest.mark.parametrize("M,K,N", [(48, 2304, 1), (48, 2304, 4), (80, 1280, 5),
                                   (272, 2560, 17), (160, 9216, 64), (64, 9216, 127),
                                   (336, 512, 128), (512, 768, 200)])
@pytest.mark.parametrize("fn", ["gemv", "gemm"])
@pytest.mark.parametrize("ydt", [bt.BT_I32, bt.BT_BF16, bt.BT_F32])
def test_matmul_paths(M, K, N, fn, ydt):
    print(f"canary {fn} M={M} K={K} N={N} ydt={ydt}", flush=True)
    w = _weights(M, K, M + K + N)
    x = W.activations(N, K, "normal", N + 7, "bf16")
    ref_packed, _ = oracle.pack(w.numpy(), 0.02)
    xq, xs, xsum = oracle.quant_act(x_for_oracle(x))
    acc = oracle.matmul_i32(ref_packed, M, K, xq)
    packed = bt.pack(w.to(DEV), 0.02)
    dq = [torch.from_numpy(a).to(DEV) for a in (xq, xs, xsum)]
    g = Guarded((N, M), TORCH_DT[ydt])
    getattr(bt, fn)(packed, M, K, *dq, ydt, y=g.t)
    torch.cuda.synchronize()
    g.check(f"{fn} M={M} K={K} N={N}")
    check_projection(packed, ref_packed, M, K, xq, xs, acc, g.t, ydt, None, f"{fn} N={N}")


# Prefill stores: bf16 output with a workgroup's 256 rows in one projection
# (results staged in LDS, whole-row stores) and, for the same call, a
# projection whose last workgroup tile is partial (per-lane stores).
@pytest.mark.parametrize("N", [130, 2048])
def test_prefill_both_store_paths_in_one_layer(N):
    shapes = ((512, 512), (64, 512), (64, 512), (768, 256), (336, 512), (336, 512),
              (512, 1280))
    wl = W.Workload(name="canary_prefill", index=9, description="", shapes=shapes,
                    layers=1, batches=(N,), x_dtype="bf16", y_dtype="bf16",
                    weight_dist="p0_0.4", act_dist="student_t4")
    ws = W.layer_weights(wl, 0)
    packed = [bt.pack(w.to(DEV), s) for (w, s) in ws]
    L = bt.Layer(packed, shapes)
    xs = W.layer_inputs(wl, 0, N)
    quant = [oracle.quant_act(x_for_oracle(x)) for x in xs]
    for ydt in (bt.BT_BF16, bt.BT_I32):
        gs = [Guarded((N, M), TORCH_DT[ydt]) for (M, _) in shapes]
        L.forward([x.to(DEV) for x in xs], y_dtype=ydt, ys=[g.t for g in gs])
        torch.cuda.synchronize()
        for p, ((w, s), (M, K)) in enumerate(zip(ws, shapes)):
            gs[p].check(f"prefill {wl.proj_names[p]} N={N} ydt={ydt}")
            ref_packed, _ = oracle.pack(w.numpy(), s)
            xq, xsc, _ = quant[wl.proj_input[p]]
            rows = np.r_[np.arange(0, M, 7), M - 1]
            acc = oracle.matmul_i32(ref_packed, M, K, xq, rows)
            check_projection(packed[p], ref_packed, M, K, xq, xsc, acc, gs[p].t, ydt, rows,
                             f"prefill {wl.proj_names[p]} N={N} ydt={ydt}")


@pytest.mark.parametrize("N,per_group", [(1, False), (3, False), (2, True), (8, False)])
def test_layer_driver_paths(N, per_group):
    # one launch per block at 1 and 3 tokens, per-group decode kernels with
    # fused quantization at 2, the four-group matrix-core launch at 8
    shapes = ((64, 2048), (16, 2048), (16, 2048), (32, 2048), (48, 2048), (48, 2048),
              (32, 4096))
    wl = W.Workload(name="canary_block", index=9, description="", shapes=shapes, layers=1,
                    batches=(N,), x_dtype="bf16", y_dtype="bf16", weight_dist="p0_0.4",
                    act_dist="normal")
    ws = W.layer_weights(wl, 0)
    packed = [bt.pack(w.to(DEV), s) for (w, s) in ws]
    L = bt.Layer(packed, shapes)
    xs = W.layer_inputs(wl, 0, N)
    gs = [Guarded((N, M), torch.int32) for (M, _) in shapes]
    L.forward([x.to(DEV) for x in xs], y_dtype=bt.BT_I32, ys=[g.t for g in gs],
              per_group=per_group)
    torch.cuda.synchronize()
    for p, ((w, s), (M, K)) in enumerate(zip(ws, shapes)):
        gs[p].check(f"block {wl.proj_names[p]} N={N}")
        xq, _, _ = oracle.quant_act(x_for_oracle(xs[wl.proj_input[p]]))
        ref_packed, _ = oracle.pack(w.numpy(), s)
        assert_equal(to_np(gs[p].t), oracle.matmul_i32(ref_packed, M, K, xq), f"proj {p}")


@pytest.mark.parametrize("N", [1, 5])
def test_base3_paths(N):
    M, K = 48, 3072
    w = _weights(M, K, 31)
    gp = Guarded((bt.bt_b3_bytes(M, K),), torch.uint8)
    bt.pack_b3(w.to(DEV), 0.02, out=gp.t)
    gu = Guarded((M, K), torch.int8)
    bt.unpack_b3(gp.t, M, K, out=gu.t)
    x = W.activations(N, K, "normal", 32, "bf16")
    xq, xs, xsum = oracle.quant_act(x_for_oracle(x))
    gy = Guarded((N, M), torch.int32)
    bt.gemv_b3(gp.t, M, K, *[torch.from_numpy(a).to(DEV) for a in (xq, xs, xsum)],
               bt.BT_I32, y=gy.t)
    torch.cuda.synchronize()
    for g, what in [(gp, "pack_b3"), (gu, "unpack_b3"), (gy, "gemv_b3")]:
        g.check(what)
    assert_equal(to_np(gp.t), base3.pack(w.numpy(), 0.02), "base-3 bytes")
    assert_equal(to_np(gu.t), w.numpy(), "base-3 unpack")
    ref_packed, _ = oracle.pack(w.numpy(), 0.02)
    assert_equal(to_np(gy.t), oracle.matmul_i32(ref_packed, M, K, xq), "base-3 product")


def test_interop_paths():
    M, K, block = 48, 768, 128
    w = _weights(M, K, 41)
    packed = bt.pack(w.to(DEV), 0.75)
    gd = Guarded((M, K), torch.bfloat16)
    bt.dequantize(packed, M, K, torch.bfloat16, out=gd.t)
    ge = Guarded((bt.bt_i2s_bytes(M, K),), torch.uint8)
    bt.i2s_export(packed, M, K, block, out=ge.t)
    gi = Guarded((bt.bt_packed_bytes(M, K),), torch.uint8)
    bt.i2s_import(ge.t, M, K, block, out=gi.t)
    torch.cuda.synchronize()
    for g, what in [(gd, "dequantize"), (ge, "i2s_export"), (gi, "i2s_import")]:
        g.check(what)
    ref_packed, _ = oracle.pack(w.numpy(), 0.75)
    assert_equal(to_np(gd.t), interop.to_float(w.numpy(), 0.75, "bf16"), "to_float")
    assert_equal(to_np(ge.t), interop.i2s_pack(w.numpy(), 0.75, block), "I2_S bytes")
    assert_equal(to_np(gi.t), ref_packed, "I2_S import")
