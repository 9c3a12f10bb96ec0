"""Per-layer driver (seven projections in four grouped launches) vs oracle,
on small layers and on the full-size workloads (all outputs where the oracle
is quick, seeded samples of output rows otherwise)."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt
import workloads as W
from parity import (RTOL, Guarded, as_f64, assert_equal, assert_rel_close,
                    check_projection, to_np, x_for_oracle)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
YDT = {"f32": bt.BT_F32, "bf16": bt.BT_BF16}

SMALL = W.Workload(
    name="small_layer", index=9, description="small block with every kind of tail",
    shapes=((256, 512), (64, 512), (64, 512), (512, 256), (336, 512),
            (336, 512), (512, 1280)),
    layers=1, batches=(1, 3, 8, 40, 64, 72, 90, 200), x_dtype="bf16", y_dtype="bf16",
    weight_dist="p0_0.4", act_dist="normal", outlier_frac=0.01, outlier_scale=20.0)


TORCH_DT = {bt.BT_I32: torch.int32, bt.BT_F32: torch.float32, bt.BT_BF16: torch.bfloat16}


def sample_rows(rng, M, count):
    """`count` random rows of M plus the first and the last 16-row tile (the
    projection's edges in a launch that lays several projections end to end)."""
    if count is None or count >= M:
        return None
    edges = np.r_[np.arange(16), np.arange(M - 16, M)]
    return np.unique(np.r_[rng.choice(M, count, replace=False), edges])


def forward_guarded(L, wl, xs, N, ydt, per_group=False):
    """L.forward into outputs between sentinel bands; checks the bands."""
    gs = [Guarded((N, M), TORCH_DT[ydt]) for (M, _) in wl.shapes]
    ys = L.forward(xs, y_dtype=ydt, ys=[g.t for g in gs], per_group=per_group)
    torch.cuda.synchronize()
    for p, g in enumerate(gs):
        g.check(f"{wl.name} {wl.proj_names[p]} N={N} ydt={ydt}")
    return ys


def run_layer(wl, layer, N, ydts, rows_per_proj=None, seed_rows=0):
    """Build one layer on the GPU, run the driver once per output type,
    compare every output with the oracle (all rows, or seeded samples)."""
    if isinstance(ydts, int):
        ydts = (ydts,)
    print(f"{wl.name} layer {layer} N={N} ydts={ydts}", flush=True)
    ws = W.layer_weights(wl, layer, device="cpu" if wl.layers == 1 else DEV)
    packed_gpu = [bt.pack(w.to(DEV), s) for (w, s) in ws]
    L = bt.Layer(packed_gpu, wl.shapes)
    xs = W.layer_inputs(wl, layer, N, device="cpu")
    xd = [x.to(DEV) for x in xs]
    outs = {ydt: forward_guarded(L, wl, xd, N, ydt) for ydt in ydts}
    rng = np.random.default_rng(seed_rows)
    quant = [oracle.quant_act(x_for_oracle(x)) for x in xs]
    for p, ((w, s), (M, K)) in enumerate(zip(ws, wl.shapes)):
        ref_packed, _ = oracle.pack(w.cpu().numpy(), s)
        assert_equal(to_np(packed_gpu[p]), ref_packed, f"packed {wl.proj_names[p]}")
        xq, xsc, _ = quant[wl.proj_input[p]]
        rows = sample_rows(rng, M, rows_per_proj)
        acc = oracle.matmul_i32(ref_packed, M, K, xq, rows)
        for ydt, ys in outs.items():
            check_projection(packed_gpu[p], ref_packed, M, K, xq, xsc, acc, ys[p], ydt,
                             rows, f"{wl.name} layer {layer} {wl.proj_names[p]} N={N} ydt={ydt}")
    return outs[ydts[0]]


@pytest.mark.parametrize("N", SMALL.batches)
@pytest.mark.parametrize("ydt", [bt.BT_I32, bt.BT_F32, bt.BT_BF16])
def test_small_layer(N, ydt):
    run_layer(SMALL, 0, N, ydt)


def test_small_layer_f32_inputs():
    wl = W.Workload(**{**SMALL.__dict__, "x_dtype": "f32"})
    run_layer(wl, 0, 5, bt.BT_F32)


# Row counts give ragged 256-row tiles in every group; three K values; 700
# tokens leave the XCD tile order a short last chunk of token tiles.
STREAM = W.Workload(
    name="prefill_groups", index=12, description="four groups of different K in one launch",
    shapes=((272, 2304), (48, 2304), (48, 2304), (2304, 1024), (1040, 2304), (1040, 2304),
            (2304, 3328)),
    layers=1, batches=(128, 257, 700, 1000), x_dtype="bf16", y_dtype="bf16",
    weight_dist="p0_0.4", act_dist="student_t4")


@pytest.mark.parametrize("N", STREAM.batches)
def test_prefill_four_groups_equal_per_group(N):
    """The four groups' tiles in one launch (largest K first, each group's
    workgroups a multiple of the XCD count) give exactly the outputs of one
    prefill launch per group, in every store path and on repeated calls."""
    ws = W.layer_weights(STREAM, 0)
    packed = [bt.pack(w.to(DEV), s) for (w, s) in ws]
    L = bt.Layer(packed, STREAM.shapes)
    xs = [x.to(DEV) for x in W.layer_inputs(STREAM, 0, N)]
    for ydt in (bt.BT_BF16, bt.BT_I32, bt.BT_F32, bt.BT_BF16):
        a = forward_guarded(L, STREAM, xs, N, ydt)
        b = L.forward(xs, y_dtype=ydt, per_group=True)
        for p in range(bt.BT_LAYER_PROJ):
            assert torch.equal(a[p], b[p]), (N, ydt, p)


def test_prefill_short_last_chunk_against_oracle():
    # 700 tokens: 11 token tiles in chunks of 2, the last chunk one tile;
    # exact int32 sums on sampled rows of every projection, bf16 too
    run_layer(STREAM, 0, 700, (bt.BT_I32, bt.BT_BF16), rows_per_proj=64, seed_rows=700)


def test_layer_matches_separate_calls():
    wl = SMALL
    N = 17
    ws = W.layer_weights(wl, 0)
    packed = [bt.pack(w.to(DEV), s) for (w, s) in ws]
    L = bt.Layer(packed, wl.shapes)
    xs = [x.to(DEV) for x in W.layer_inputs(wl, 0, N)]
    ys = L.forward(xs, y_dtype=bt.BT_BF16)
    for p, (M, K) in enumerate(wl.shapes):
        xq, s, sm = bt.quant_act(xs[wl.proj_input[p]])
        y = bt.gemv(packed[p], M, K, xq, s, sm, bt.BT_BF16)
        assert torch.equal(y, ys[p])


# ------------------------------------------------- full-size workloads ----

def test_workload_gemv_2560():
    wl = W.GEMV_2560
    for ydt in (bt.BT_I32, bt.BT_F32):
        w, s = W.layer_weights(wl, 0)[0]
        assert s == 0.02
        M, K = wl.shapes[0]
        x = W.layer_inputs(wl, 0, 1)[0]
        packed = bt.pack(w.to(DEV), s)
        xq, xs, xsum = bt.quant_act(x.to(DEV))
        y = bt.gemv(packed, M, K, xq, xs, xsum, ydt)
        ref_packed, _ = oracle.pack(w.numpy(), s)
        ref = oracle.forward(ref_packed, M, K, x.numpy())
        assert_equal(to_np(packed), ref_packed, "packed")
        assert_equal(to_np(xq), ref["xq"], "xq")
        if ydt == bt.BT_I32:
            assert_equal(to_np(y), ref["acc"], "acc")
        else:
            assert_rel_close(as_f64(y), ref["y"], 1e-6, "y")


def test_workload_layer2b_n1():
    run_layer(W.LAYER2B_N1, 0, 1, (bt.BT_I32, bt.BT_BF16, bt.BT_F32))


def test_workload_layer2b_n64():
    run_layer(W.LAYER2B_N64, 0, 64, (bt.BT_I32, bt.BT_BF16, bt.BT_F32))


def test_workload_prefill_sampled_rows():
    run_layer(W.PREFILL2B_N2048, 0, 2048, (bt.BT_I32, bt.BT_BF16), rows_per_proj=64,
              seed_rows=1)


# The 70B-class block: exact int32 sums on 256 sampled rows per projection
# plus each projection's first and last row tile (the one-launch kernel at 1
# token with its balanced two-class schedule, the matrix-core decode at 8,
# and at 33 and 64 tokens where the down projection runs in K phases), and
# the bf16 outputs of the same call.
@pytest.mark.parametrize("layer", [0, 79])
@pytest.mark.parametrize("N", [1, 8])
def test_workload_stream70b_sampled_rows(layer, N):
    run_layer(W.STREAM70B, layer, N, (bt.BT_I32, bt.BT_BF16), rows_per_proj=256,
              seed_rows=layer + N)


# 24 tokens: two token groups on the matrix-core decode with cached weight
# loads; 33 and 64: the prefill kernel.
@pytest.mark.parametrize("N", [24, 33, 64])
def test_workload_stream70b_many_tokens(N):
    run_layer(W.STREAM70B, 0, N, (bt.BT_I32,), rows_per_proj=64, seed_rows=N)


def test_determinism():
    outs = [run_layer(SMALL, 0, 64, bt.BT_BF16) for _ in range(3)]
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    for a, b in zip(outs[0], outs[2]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("N", [8, 64, 200])
def test_quantize_all_inputs_at_once_equals_per_group(N):
    """The driver quantizes the four inputs in one launch unless asked for
    per-group launches; both orders give identical outputs."""
    wl = SMALL
    ws = W.layer_weights(wl, 0)
    packed = [bt.pack(w.to(DEV), s) for (w, s) in ws]
    L = bt.Layer(packed, wl.shapes)
    xs = [x.to(DEV) for x in W.layer_inputs(wl, 0, N)]
    for ydt in (bt.BT_I32, bt.BT_BF16):
        a = L.forward(xs, y_dtype=ydt)
        b = L.forward(xs, y_dtype=ydt, per_group=True)
        for p in range(7):
            assert torch.equal(a[p], b[p]), (N, ydt, p)


# ------------------------------------------------- base-3 weights ----------

# every K >= 4096 and a multiple of 1024: one launch at 1 and 2 tokens (the
# codes of two tokens fill the 80 KiB next to the decode table exactly),
# quantization + one base-3 product per projection from 3 tokens on
B3_BLOCK = W.Workload(
    name="b3_block", index=9, description="block for the base-3 layer path",
    shapes=((64, 8192), (16, 8192), (16, 8192), (48, 8192), (80, 8192),
            (80, 8192), (32, 16384)),
    layers=1, batches=(1, 2, 3, 5), x_dtype="bf16", y_dtype="bf16",
    weight_dist="p0_0.4", act_dist="normal", outlier_frac=0.005, outlier_scale=30.0)


def run_layer_b3(wl, layer, N, ydts, rows_per_proj=None, seed_rows=0, per_group=False):
    """The driver on base-3 weights against the oracle's product."""
    if isinstance(ydts, int):
        ydts = (ydts,)
    print(f"base-3 {wl.name} layer {layer} N={N} ydts={ydts}", flush=True)
    ws = W.layer_weights(wl, layer, device="cpu" if wl.layers == 1 else DEV)
    packed = [bt.pack_b3(w.to(DEV), s) for (w, s) in ws]
    L = bt.Layer(packed, wl.shapes, base3=True)
    xs = W.layer_inputs(wl, layer, N, device="cpu")
    xd = [x.to(DEV) for x in xs]
    outs = {ydt: forward_guarded(L, wl, xd, N, ydt, per_group) for ydt in ydts}
    rng = np.random.default_rng(seed_rows)
    quant = [oracle.quant_act(x_for_oracle(x)) for x in xs]
    for p, ((w, s), (M, K)) in enumerate(zip(ws, wl.shapes)):
        ref_packed, _ = oracle.pack(w.cpu().numpy(), s)
        xq, xsc, _ = quant[wl.proj_input[p]]
        rows = sample_rows(rng, M, rows_per_proj)
        acc = oracle.matmul_i32(ref_packed, M, K, xq, rows)
        for ydt, ys in outs.items():
            check_projection(packed[p], ref_packed, M, K, xq, xsc, acc, ys[p], ydt, rows,
                             f"base-3 {wl.name} layer {layer} {wl.proj_names[p]} N={N} ydt={ydt}")
    return outs[ydts[0]]


@pytest.mark.parametrize("N", B3_BLOCK.batches)
@pytest.mark.parametrize("ydt", [bt.BT_I32, bt.BT_F32, bt.BT_BF16])
def test_base3_layer(N, ydt):
    print(f"base-3 layer N={N} ydt={ydt}", flush=True)
    run_layer_b3(B3_BLOCK, 0, N, ydt)


@pytest.mark.parametrize("N", [1, 3])
def test_base3_layer_per_group(N):
    run_layer_b3(B3_BLOCK, 0, N, bt.BT_I32, per_group=True)


def test_base3_layer_shortest_one_launch_rows():
    # K = 4096 everywhere: one tile column per wave of the K split; 3 and 4
    # tokens also fit one launch here (the four-token instantiation)
    wl = W.Workload(**{**B3_BLOCK.__dict__, "name": "b3_4096",
                       "shapes": ((64, 4096), (16, 4096), (16, 4096), (48, 4096),
                                  (80, 4096), (80, 4096), (32, 4096))})
    for N in (1, 2, 3, 4):
        run_layer_b3(wl, 0, N, (bt.BT_I32, bt.BT_BF16))


def test_base3_layer_short_rows():
    # K = 1024..3072: never one launch; quantization + base-3 products
    wl = W.Workload(**{**B3_BLOCK.__dict__, "name": "b3_short",
                       "shapes": ((64, 2048), (16, 2048), (16, 2048), (48, 1024),
                                  (80, 2048), (80, 2048), (32, 3072))})
    for N in (1, 4, 9):
        run_layer_b3(wl, 0, N, bt.BT_I32)


@pytest.mark.parametrize("N", [1, 2, 5])
def test_base3_layer_equals_two_bit_layer(N):
    # same weights in both formats: identical bf16 outputs, bit for bit
    wl = B3_BLOCK
    ws = W.layer_weights(wl, 0)
    L2 = bt.Layer([bt.pack(w.to(DEV), s) for (w, s) in ws], wl.shapes)
    L3 = bt.Layer([bt.pack_b3(w.to(DEV), s) for (w, s) in ws], wl.shapes, base3=True)
    xs = [x.to(DEV) for x in W.layer_inputs(wl, 0, N)]
    a = L2.forward(xs, y_dtype=bt.BT_BF16)
    b = L3.forward(xs, y_dtype=bt.BT_BF16)
    for p in range(7):
        assert torch.equal(a[p], b[p]), (N, p)


@pytest.mark.parametrize("layer", [0, 79])
def test_workload_stream70b_base3_sampled_rows(layer):
    # the 70B-class block in base-3 bytes at one token (one launch): exact
    # int32 sums on 256 sampled rows per projection plus its edge tiles, and
    # the bf16 outputs
    run_layer_b3(W.STREAM70B, layer, 1, (bt.BT_I32, bt.BT_BF16), rows_per_proj=256,
                 seed_rows=layer)
