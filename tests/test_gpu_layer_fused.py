"""The one-launch block kernel (all seven projections, the four inputs
quantized in its prologue) against the oracle and, bit for bit, against the
per-group launches of the same driver."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt
import workloads as W
from parity import assert_equal, check_projection, to_np, x_for_oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"

# K >= 2048 everywhere, so the block runs as one launch for 1..4 tokens.
# Row counts give ragged tile totals (odd, and not a multiple of the grid).
SPLIT8 = W.Workload(
    name="fused_split8", index=10, description="K split over 8 waves (min K 2048)",
    shapes=((272, 2304), (48, 2304), (48, 2304), (2304, 2048), (1040, 2304),
            (1040, 2304), (2304, 4352)),
    layers=1, batches=(1, 2, 3, 4), x_dtype="bf16", y_dtype="bf16",
    weight_dist="p0_0.4", act_dist="normal", outlier_frac=0.01, outlier_scale=20.0)
SPLIT16 = W.Workload(
    name="fused_split16", index=11,
    description="K split over 16 waves (min K 4096), few tiles; at 4 tokens the input "
                "chunks exactly fill the prologue's registers",
    shapes=((64, 4096), (16, 4096), (16, 4096), (112, 4096), (80, 4096), (80, 4096),
            (48, 4096)),
    layers=1, batches=(1, 2, 3, 4), x_dtype="bf16", y_dtype="bf16",
    weight_dist="uniform", act_dist="student_t4", outlier_frac=0.005, outlier_scale=30.0)


def build(wl):
    ws = W.layer_weights(wl, 0)
    packed = [bt.pack(w.to(DEV), s) for (w, s) in ws]
    return ws, packed, bt.Layer(packed, wl.shapes)


@pytest.mark.parametrize("wl", [SPLIT8, SPLIT16], ids=lambda w: w.name)
@pytest.mark.parametrize("N", [1, 2, 3, 4])
def test_fused_block_exact_and_equal_to_per_group(wl, N):
    ws, packed, L = build(wl)
    assert bt.bt_layer_one_launch(L.c, N, bt.BT_BF16) == 1
    xs = W.layer_inputs(wl, 0, N)
    xd = [x.to(DEV) for x in xs]
    quant = [oracle.quant_act(x_for_oracle(x)) for x in xs]
    for ydt in (bt.BT_I32, bt.BT_F32, bt.BT_BF16):
        fused = L.forward(xd, y_dtype=ydt)
        grouped = L.forward(xd, y_dtype=ydt, per_group=True)
        torch.cuda.synchronize()
        for p, ((w, s), (M, K)) in enumerate(zip(ws, wl.shapes)):
            assert torch.equal(fused[p], grouped[p]), (wl.name, N, ydt, p)
            if ydt == bt.BT_BF16:
                continue
            ref_packed, _ = oracle.pack(w.numpy(), s)
            xq, xsc, _ = quant[wl.proj_input[p]]
            acc = oracle.matmul_i32(ref_packed, M, K, xq, None)
            check_projection(packed[p], ref_packed, M, K, xq, xsc, acc, fused[p], ydt,
                             None, f"{wl.name} {wl.proj_names[p]} N={N}")


def test_fused_block_layer2b_all_tokens():
    """The 2B-class block: one launch up to 3 tokens; at 4 the four-group
    matrix-core launch (faster there) -- equal to per-group launches either
    way."""
    wl = W.LAYER2B_N1
    ws, packed, L = build(wl)
    for N in (1, 3, 4):
        assert bt.bt_layer_one_launch(L.c, N, bt.BT_BF16) == (1 if N <= 3 else 0)
        xs = [x.to(DEV) for x in W.layer_inputs(wl, 0, N)]
        fused = L.forward(xs, y_dtype=bt.BT_I32)
        grouped = L.forward(xs, y_dtype=bt.BT_I32, per_group=True)
        for a, b in zip(fused, grouped):
            assert torch.equal(a, b)


def test_fused_block_repeated_calls_and_zero_token():
    """Back-to-back calls on one stream reuse nothing between launches; a
    token whose inputs are all zero gives zero outputs."""
    wl = SPLIT8
    _, _, L = build(wl)
    xs = [x.to(DEV) for x in W.layer_inputs(wl, 0, 3)]
    xs[2][1] = 0
    first = L.forward(xs, y_dtype=bt.BT_F32)
    for _ in range(3):
        again = L.forward(xs, y_dtype=bt.BT_F32)
    for a, b in zip(first, again):
        assert torch.equal(a, b)
    assert not to_np(first[4])[1].any() and not to_np(first[5])[1].any()


@pytest.mark.parametrize("wl", [SPLIT8, SPLIT16], ids=lambda w: w.name)
def test_fused_block_tiny_token_infinite_reciprocal(wl):
    """A token whose 127 / amax overflows (inputs ~1e-39): inv = +inf, so the
    codes are 127 * sign(x) (0 * inf taken as 0) on both launch structures
    and match the oracle."""
    ws, packed, L = build(wl)
    xs = W.layer_inputs(wl, 0, 2)
    xs[0] = xs[0].float()
    xs[0][1] *= 1e-39
    xs[0] = xs[0].to(torch.bfloat16)
    xd = [x.to(DEV) for x in xs]
    fused = L.forward(xd, y_dtype=bt.BT_I32)
    grouped = L.forward(xd, y_dtype=bt.BT_I32, per_group=True)
    xq, _, _ = oracle.quant_act(x_for_oracle(xs[0]))
    assert set(np.unique(xq[1])) <= {-127, 0, 127}
    for p in range(3):  # q, k, v read input 0
        M, K = wl.shapes[p]
        ref_packed, _ = oracle.pack(ws[p][0].numpy(), ws[p][1])
        assert_equal(to_np(fused[p]), oracle.matmul_i32(ref_packed, M, K, xq, None), f"proj {p}")
    for a, b in zip(fused, grouped):
        assert torch.equal(a, b)
