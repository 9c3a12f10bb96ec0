"""Base-3 (B3T1024) format on the GPU vs the oracle: packed bytes and
unpacked weights identical, decode products bit-exact in int32 and within
1e-6 (fp32) / 1e-2 (bf16) relative, at shapes that cover every K split of
the kernel, both activation sources (LDS-staged and read from global memory),
token passes of four with ragged remainders, and the full 70B-class sizes
(sampled rows)."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt
import workloads as W
from oracle import base3 as b3
from parity import RTOL, as_f64, assert_equal, assert_rel_close, to_np, x_for_oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


@pytest.mark.parametrize("M,K", [(16, 1024), (48, 2048), (80, 3072), (256, 7168)])
def test_pack_and_unpack_exact(M, K):
    print(f"b3 pack {M}x{K}", flush=True)
    w = W.ternary_weights(M, K, "uniform", M + K)
    ref = b3.pack(w.numpy(), 0.0275)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    packed = bt.pack_b3(w.to(DEV), 0.0275, invalid_count=cnt)
    assert_equal(to_np(packed), ref, "B3 packed bytes")
    assert int(cnt.item()) == 0
    back = bt.unpack_b3(torch.from_numpy(ref).to(DEV), M, K)
    assert_equal(to_np(back), w.numpy(), "B3 unpack of the oracle's bytes")


def test_pack_invalid_values_clamped_and_counted():
    M, K = 32, 1024
    w = W.ternary_weights(M, K, "uniform", 5)
    w[0, 0] = 7
    w[5, 300] = -128
    w[31, 1023] = 2
    w[17, 48] = -2
    clamped = w.clamp(-1, 1)
    cnt = torch.full((1,), 3, dtype=torch.int32, device=DEV)  # the kernel adds
    packed = bt.pack_b3(w.to(DEV), 1.0, invalid_count=cnt)
    assert_equal(to_np(packed), b3.pack(clamped.numpy(), 1.0), "B3 packed bytes")
    assert int(cnt.item()) == 3 + 4


def _weights(M, K, seed, dist="p0_0.4"):
    """(int8 W, the oracle's 2-bit bytes -- the product's definition -- and
    the oracle's B3 bytes on the GPU)."""
    w = W.ternary_weights(M, K, dist, seed)
    s = 0.02 + (seed % 7) * 0.001
    ref2, _ = oracle.pack(w.numpy(), s)
    return w, ref2, torch.from_numpy(b3.pack(w.numpy(), s)).to(DEV)


def _tokens(ref2, M, K, N, seed):
    x = W.activations(N, K, "normal", seed, "bf16", 0.01, 20.0)
    ref = oracle.forward(ref2, M, K, x_for_oracle(x))
    xq, xs, xsum = bt.quant_act(x.to(DEV))
    return ref, xq, xs, xsum


def _gemv_case(M, K, N, seed):
    _, ref2, packed = _weights(M, K, seed)
    ref, xq, xs, xsum = _tokens(ref2, M, K, N, seed + 1)
    return ref, packed, xq, xs, xsum


# K = 1024 (one tile column: no K split), 2048 (split 2), 5120 (split 4,
# uneven), 8192 (split 8), 28672 (3-4 tile columns per wave; codes of two
# tokens still staged in LDS, four read from global memory)
@pytest.mark.parametrize("M,K", [(16, 1024), (64, 2048), (48, 5120), (1040, 8192),
                                 (112, 28672)])
def test_gemv_int32_exact(M, K):
    _, ref2, packed = _weights(M, K, M * 31 + K)
    for N in (1, 2, 3, 4, 5, 9):
        print(f"b3 gemv {M}x{K} N={N}", flush=True)
        ref, xq, xs, xsum = _tokens(ref2, M, K, N, M + K + N)
        y = bt.gemv_b3(packed, M, K, xq, xs, xsum, bt.BT_I32)
        assert_equal(to_np(y), ref["acc"], f"B3 gemv M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K", [(32768, 1024), (32768, 3072)])
def test_gemv_tall_matrices_whole_row_tiles(M, K):
    # 2048 row tiles: enough for the shape in which every wave owns whole row
    # tiles (no K split, no cross-wave reduction); the weights are packed on
    # the GPU (their bytes are pinned to the oracle's above) and every output
    # is compared with the oracle's product
    w = W.ternary_weights(M, K, "p0_0.4", M + K)
    ref2, _ = oracle.pack(w.numpy(), 0.025)
    packed = bt.pack_b3(w.to(DEV), 0.025)
    for N in (1, 2, 3, 4, 5):
        print(f"b3 gemv tall {M}x{K} N={N}", flush=True)
        ref, xq, xs, xsum = _tokens(ref2, M, K, N, 3 * N + K)
        y = bt.gemv_b3(packed, M, K, xq, xs, xsum, bt.BT_I32)
        assert_equal(to_np(y), ref["acc"], f"B3 gemv M={M} K={K} N={N}")
        y = bt.gemv_b3(packed, M, K, xq, xs, xsum, bt.BT_BF16)
        assert_rel_close(as_f64(y), ref["y"], RTOL[bt.BT_BF16], f"B3 gemv bf16 N={N}")


@pytest.mark.parametrize("ydt", [bt.BT_F32, bt.BT_BF16])
def test_gemv_float_within_tolerance(ydt):
    for (M, K, N) in [(48, 2048, 1), (80, 3072, 2), (1040, 8192, 4), (32, 4096, 7)]:
        ref, packed, xq, xs, xsum = _gemv_case(M, K, N, M + 3 * K + N)
        y = bt.gemv_b3(packed, M, K, xq, xs, xsum, ydt)
        assert_rel_close(as_f64(y), ref["y"], RTOL[ydt], f"B3 gemv {M}x{K} N={N}")


def test_gemv_matches_the_two_bit_path_bitwise():
    # same weights in both formats: identical float outputs, bit for bit
    M, K = 208, 4096
    for N in (1, 2, 4):
        w = W.ternary_weights(M, K, "p0_0.4", 900 + N)
        x = W.activations(N, K, "normal", 901 + N, "bf16", 0.01, 20.0).to(DEV)
        xq, xs, xsum = bt.quant_act(x)
        p2 = bt.pack(w.to(DEV), 0.031)
        p3 = bt.pack_b3(w.to(DEV), 0.031)
        for ydt in (bt.BT_F32, bt.BT_BF16):
            a = to_np(bt.gemv(p2, M, K, xq, xs, xsum, ydt))
            b = to_np(bt.gemv_b3(p3, M, K, xq, xs, xsum, ydt))
            assert_equal(b.view(np.uint32) if ydt == bt.BT_F32 else b,
                         a.view(np.uint32) if ydt == bt.BT_F32 else a, f"N={N} ydt={ydt}")


def test_gemv_extreme_activations_and_weights():
    # all weights +1 or -1 and activations at +-127: the largest sums
    M, K = 32, 8192
    for fill in (1, -1):
        w = torch.full((M, K), fill, dtype=torch.int8)
        xq = torch.full((2, K), 127, dtype=torch.int8)
        xq[1] = -127
        xs = torch.tensor([1.0, 2.0])
        xsum = xq.sum(dim=1, dtype=torch.int32)
        packed = torch.from_numpy(b3.pack(w.numpy(), 0.5)).to(DEV)
        y = bt.gemv_b3(packed, M, K, xq.to(DEV), xs.to(DEV), xsum.to(DEV), bt.BT_I32)
        want = np.array([[fill * 127 * K] * M, [-fill * 127 * K] * M], dtype=np.int32)
        assert_equal(to_np(y), want, f"fill {fill}")


def test_gemv_zero_tokens_is_a_no_op():
    M, K = 16, 1024
    packed = torch.from_numpy(b3.pack(np.zeros((M, K), np.int8), 1.0)).to(DEV)
    y = torch.full((1, M), 7, dtype=torch.int32, device=DEV)
    e = torch.empty((0, K), dtype=torch.int8, device=DEV)
    f = torch.empty(0, dtype=torch.float32, device=DEV)
    i = torch.empty(0, dtype=torch.int32, device=DEV)
    bt.bt_ternary_gemv_b3(packed, M, K, e, f, i, 0, y, bt.BT_I32)
    torch.cuda.synchronize()
    assert (y == 7).all()


def test_gemv_longest_rows_from_global_memory():
    # K = 131072 (the largest multiple of 1024 allowed): even one token's
    # codes do not fit in LDS beside the table
    M, K, N = 32, 131072, 1
    ref, packed, xq, xs, xsum = _gemv_case(M, K, N, 77)
    y = bt.gemv_b3(packed, M, K, xq, xs, xsum, bt.BT_I32)
    assert_equal(to_np(y), ref["acc"], "K = 131072")


@pytest.mark.parametrize("M,K", [(28672, 8192), (8192, 28672)])
def test_full_size_sampled(M, K):
    # the 70B-class gate/up and down matrices in the shape the benchmark
    # times: GPU packing (sampled rows decoded by the oracle) and one- and
    # four-token products (sampled rows of the oracle's product)
    print(f"b3 full size {M}x{K}", flush=True)
    w = W.ternary_weights(M, K, "p0_0.4", 4242, device=DEV)
    packed = bt.pack_b3(w, 0.0213)
    rows = np.sort(np.random.default_rng(M).choice(M, 48, replace=False))
    got, s = b3.unpack(to_np(packed), M, K, rows=rows)
    assert_equal(got, to_np(w)[rows], "sampled rows of the GPU-packed bytes")
    assert s == np.float32(0.0213)
    ref2, _ = oracle.pack(to_np(w), 0.0213)
    for N in (1, 4):
        x = W.activations(N, K, "normal", 4243 + N, "bf16", 0.005, 30.0)
        xq_ref, _, _ = oracle.quant_act(x_for_oracle(x))
        xq, xs, xsum = bt.quant_act(x.to(DEV))
        y = to_np(bt.gemv_b3(packed, M, K, xq, xs, xsum, bt.BT_I32))
        acc = oracle.matmul_i32(ref2, M, K, xq_ref, rows)
        assert_equal(y[:, rows], acc, f"sampled rows N={N}")
