"""bt_ternary_linear (quantization and product in one call) against the CPU
oracle and against the two-call path (bt_quant_act, then bt_ternary_gemv or
bt_ternary_gemm): exact int32 sums, float outputs bit for bit equal to the
two-call path and within 1e-6 (fp32) / 1e-2 (bf16) of the oracle, on the one-
launch path (the decode kernel quantizes the tokens in its prologue) and on
the workspace path, with sentinel bands around every output."""
import pytest
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt
import workloads as W
from parity import RTOL, as_f64, assert_equal, assert_rel_close, guarded, to_np, x_for_oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
DT = {"f32": bt.BT_F32, "bf16": bt.BT_BF16}

# (M, K, N, x dtype, one launch?)
CASES = [
    (2560, 2560, 1, "f32", 1),     # the single 2560 x 2560 GEMV
    (16, 256, 1, "bf16", 1),       # one tile
    (48, 32768, 1, "bf16", 1),     # longest bf16 row the prologue holds
    (48, 16384, 1, "f32", 1),      # longest fp32 row the prologue holds
    (48, 16640, 1, "f32", 0),      # one block longer: through the workspace
    (48, 65536, 1, "bf16", 0),
    (208, 2304, 3, "bf16", 1),     # three tokens, ragged token group
    (4096, 2560, 8, "bf16", 0),    # matrix-core decode
    (80, 1280, 130, "bf16", 0),    # prefill kernel
]


def _inputs(M, K, N, xdt, seed):
    w = W.ternary_weights(M, K, "p0_0.4", seed)
    x = W.activations(N, K, "normal", seed + 1, xdt, 0.01, 20.0)
    scale = 0.02 + (seed % 5) * 0.001
    ref_packed, _ = oracle.pack(w.numpy(), scale)
    ref = oracle.forward(ref_packed, M, K, x_for_oracle(x))
    return bt.pack(w.to(DEV), scale), x.to(DEV), ref


@pytest.mark.parametrize("M,K,N,xdt,one", CASES)
def test_linear_against_oracle_and_two_calls(M, K, N, xdt, one):
    assert bt.bt_linear_one_launch(N, M, K, DT[xdt]) == one
    packed, x, ref = _inputs(M, K, N, xdt, M + 3 * K + N)
    xq, xs, xsum = bt.quant_act(x)
    two = bt.gemv if N < bt.BT_PREFILL_MIN_N else bt.gemm
    for ydt in (bt.BT_I32, bt.BT_F32, bt.BT_BF16):
        g, y = guarded((N, M), {bt.BT_I32: torch.int32, bt.BT_F32: torch.float32,
                                bt.BT_BF16: torch.bfloat16}[ydt])
        bt.linear(packed, M, K, x, ydt, y=y)
        torch.cuda.synchronize()
        g.check(f"linear {M}x{K} N={N} y={ydt}")
        what = f"linear {M}x{K} N={N} {xdt} y={ydt}"
        if ydt == bt.BT_I32:
            assert_equal(to_np(y), ref["acc"], what)
        else:
            assert_rel_close(as_f64(y), ref["y"], RTOL[ydt], what)
        y2 = two(packed, M, K, xq, xs, xsum, ydt)
        assert_equal(to_np(y), to_np(y2), what + " vs two calls")


def test_linear_workspace_rules():
    M, K, N = 4096, 2560, 8
    packed, x, ref = _inputs(M, K, N, "bf16", 11)
    need = bt.bt_linear_workspace_bytes(N, K)
    assert need == 20480 + 256 + 256
    y = torch.empty((N, M), dtype=torch.int32, device=DEV)
    small = torch.empty(need - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(bt.BtError, match="workspace"):
        bt.linear(packed, M, K, x, bt.BT_I32, workspace=small, y=y)
    # a workspace with stale contents, used twice
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
    for _ in range(2):
        y.fill_(-7)
        bt.linear(packed, M, K, x, bt.BT_I32, workspace=ws, y=y)
        assert_equal(to_np(y), ref["acc"], "linear with a reused workspace")
    # the one-launch path ignores the workspace (NULL is fine)
    packed1, x1, ref1 = _inputs(2560, 2560, 1, "f32", 12)
    y1 = torch.empty((1, 2560), dtype=torch.int32, device=DEV)
    bt.bt_ternary_linear(packed1, 2560, 2560, x1, bt.BT_F32, 1, y1, bt.BT_I32, None, 0)
    assert_equal(to_np(y1), ref1["acc"], "one launch, no workspace")


def test_linear_zero_tokens_is_a_noop():
    M, K = 64, 512
    packed, _, _ = _inputs(M, K, 1, "f32", 13)
    bt.bt_ternary_linear(packed, M, K, None, bt.BT_F32, 0, None, bt.BT_F32, None, 0)
    torch.cuda.synchronize()


def test_linear_on_a_side_stream():
    M, K, N = 1024, 2560, 2
    packed, x, ref = _inputs(M, K, N, "bf16", 14)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = bt.linear(packed, M, K, x, bt.BT_I32, stream=s)
    s.synchronize()
    assert_equal(to_np(y), ref["acc"], "linear on a side stream")
