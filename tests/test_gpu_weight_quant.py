"""GPU weight quantizer vs the oracle: the statistic s, the divisor d and
every packed byte must be identical (the mean is exact by definition, the
codes are integer decisions)."""
import numpy as np
import pytest
import torch

import ternary_weight_quantized_bt_amd as bt
import workloads as W
from oracle import weight_quant as wq
from parity import assert_equal, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _oracle_input(w: torch.Tensor) -> np.ndarray:
    if w.dtype == torch.bfloat16:
        return w.view(torch.int16).numpy().view(np.uint16)
    return w.numpy()


def _check(w: torch.Tensor, mode: str, eps: float):
    M, K = w.shape
    print(f"weight quantizer: {M}x{K} {w.dtype} {mode} eps={eps}", flush=True)
    ref_packed, s, d = wq.quantize_weights(_oracle_input(w), mode, eps)
    packed, stats = bt.quantize_weights(w.to(DEV), mode, eps)
    torch.cuda.synchronize()
    st = to_np(stats)
    assert st[0].view(np.uint32) == np.float32(s).view(np.uint32), (st[0], s)
    assert st[1].view(np.uint32) == np.float32(d).view(np.uint32), (st[1], d)
    assert_equal(to_np(packed), ref_packed, "packed bytes")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["absmean", "absmax"])
@pytest.mark.parametrize("M,K,dist", [
    (16, 256, "normal"), (48, 768, "student_t4"), (80, 2304, "normal"),
    (64, 2560, "wide"), (32, 1024, "subnormal"), (16, 512, "ternarized")])
def test_matches_oracle(M, K, dist, mode, dtype):
    w = W.float_weights(M, K, dist, 1000 + M + K, dtype)
    _check(w, mode, 1e-5 if dist == "normal" else 0.0)


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.001, 0.05])
def test_eps(eps):
    _check(W.float_weights(48, 1280, "normal", 7), "absmean", eps)


def test_all_zero_tensor():
    w = W.float_weights(16, 256, "zeros", 0)
    _check(w, "absmean", 0.0)     # d = 0: every code is 0 (0/0)
    _check(w, "absmax", 1e-5)


def test_pre_ternarized_tensor_comes_back():
    M, K = 64, 1024
    t = W.ternary_weights(M, K, "p0_0.4", 21)
    w = W.float_weights(M, K, "ternarized", 21)
    packed, stats = bt.quantize_weights(w.to(DEV), "absmax", 0.0)
    assert np.array_equal(to_np(bt.unpack(packed, M, K)), t.numpy())
    assert to_np(stats)[1] == np.float32(0.0213)


def test_projection_sized_tensors():
    # the 2560 x 6912 down projection and a 6912 x 2560 gate of the 2B block
    for (M, K, seed) in [(2560, 6912, 3), (6912, 2560, 4)]:
        _check(W.float_weights(M, K, "normal", seed, "bf16"), "absmean", 1e-5)


def test_repeated_calls_reuse_the_workspace():
    w1 = W.float_weights(48, 768, "wide", 5)
    w2 = W.float_weights(16, 256, "normal", 6)
    ws_bytes = bt.bt_quantize_weights_workspace_bytes()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    for w in (w1, w2, w1):
        M, K = w.shape
        packed = torch.empty(bt.bt_packed_bytes(M, K), dtype=torch.uint8, device=DEV)
        stats = torch.empty(2, dtype=torch.float32, device=DEV)
        bt.bt_quantize_weights(w.to(DEV), bt.BT_F32, M, K, bt.BT_WSCALE_ABSMEAN, 0.0,
                               packed, stats, ws, ws_bytes)
        ref, s, d = wq.quantize_weights(w.numpy(), "absmean", 0.0)
        assert_equal(to_np(packed), ref, "packed bytes")
        assert to_np(stats)[0] == s


def test_without_stats_output():
    w = W.float_weights(16, 256, "normal", 8)
    ws = torch.empty(bt.bt_quantize_weights_workspace_bytes(), dtype=torch.uint8, device=DEV)
    packed = torch.empty(bt.bt_packed_bytes(16, 256), dtype=torch.uint8, device=DEV)
    bt.bt_quantize_weights(w.to(DEV), bt.BT_F32, 16, 256, bt.BT_WSCALE_ABSMEAN, 0.0,
                           packed, None, ws, ws.numel())
    ref, _, _ = wq.quantize_weights(w.numpy(), "absmean", 0.0)
    assert_equal(to_np(packed), ref, "packed bytes")


def test_full_size_gate_matrix_sampled_rows():
    # the 28672 x 8192 bf16 gate/up matrix of the 70B-class block, in the
    # configuration the benchmark times: the statistic and the divisor over
    # the whole tensor bit for bit, and 64 sampled rows of codes against the
    # oracle's RoundClip with that divisor
    M, K = 28672, 8192
    print("weight quantizer: full-size gate matrix", flush=True)
    w = W.float_weights(M, K, "normal", 77, "bf16", device=DEV)
    packed, stats = bt.quantize_weights(w, "absmean", 1e-5)
    bits = w.view(torch.int16).cpu().numpy().view(np.uint16)
    s = wq.abs_mean(bits)
    d = np.float32(s + np.float32(1e-5))
    st = to_np(stats)
    assert st[0].view(np.uint32) == np.float32(s).view(np.uint32), (st[0], s)
    assert st[1].view(np.uint32) == d.view(np.uint32), (st[1], d)
    rows = np.sort(np.random.default_rng(5).choice(M, 64, replace=False))
    got = to_np(bt.unpack(packed, M, K))[rows]
    with np.errstate(divide="ignore", invalid="ignore"):
        want = wq.round_clip(wq.as_f32(bits[rows]) / d)
    assert_equal(got, want, "sampled rows of codes")
    tail = to_np(packed[M * K // 4: M * K // 4 + 4])
    assert tail.view(np.float32)[0] == d  # the stored scale is the divisor
