"""Pins of the oracle's integer product and dequantization.

The expected values come from routes other than the oracle's own formula:
the add / subtract / skip rule of the ternary contraction figure, closed
forms for special weight matrices, and a float64 library matmul.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand_w(rng, M, K, p0=0.4):
    u = rng.random((M, K))
    return ((u >= 1 - (1 - p0) / 2).astype(np.int8)
            - (u < (1 - p0) / 2).astype(np.int8))


@pytest.mark.parametrize("M,K,N", [(16, 256, 1), (48, 512, 3), (64, 768, 17)])
def test_add_subtract_skip_identity(M, K, N):
    # "LLM Quantization Paradigms…", section 5, figure "BitNet b1.58 Ternary
    # Matrix Multiplication": +1 adds the activation, -1 subtracts it, 0 skips.
    rng = np.random.default_rng(M * K + N)
    w = _rand_w(rng, M, K)
    xq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    p, _ = oracle.pack(w, 0.1)
    acc = oracle.matmul_i32(p, M, K, xq)
    x64 = xq.astype(np.int64)
    plus = np.stack([(x64 * (w[m] == 1)).sum(1) for m in range(M)], 1)
    minus = np.stack([(x64 * (w[m] == -1)).sum(1) for m in range(M)], 1)
    np.testing.assert_array_equal(acc, plus - minus)


def test_offset_identity():
    # sum_k (code - 1) * x == sum_k code * x - sum_k x with code = w + 1
    rng = np.random.default_rng(5)
    M, K, N = 32, 512, 4
    w = _rand_w(rng, M, K)
    xq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    p, _ = oracle.pack(w, 1.0)
    acc = oracle.matmul_i32(p, M, K, xq)
    codes = (w.astype(np.int64) + 1)
    expect = xq.astype(np.int64) @ codes.T - xq.astype(np.int64).sum(1, keepdims=True)
    np.testing.assert_array_equal(acc, expect)


@pytest.mark.parametrize("value", [0, 1, -1])
def test_constant_weights(value):
    rng = np.random.default_rng(2)
    M, K, N = 16, 512, 5
    xq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    p, _ = oracle.pack(np.full((M, K), value, np.int8), 1.0)
    acc = oracle.matmul_i32(p, M, K, xq)
    col = value * xq.astype(np.int64).sum(1)
    np.testing.assert_array_equal(acc, np.repeat(col[:, None], M, 1))


def test_permutation_rows_gather():
    # one +1 per row at column perm[m]: the product gathers those columns
    rng = np.random.default_rng(9)
    M, K, N = 32, 256, 3
    perm = rng.permutation(K)[:M]
    w = np.zeros((M, K), np.int8)
    w[np.arange(M), perm] = 1
    xq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    acc = oracle.matmul_i32(oracle.pack(w, 1.0)[0], M, K, xq)
    np.testing.assert_array_equal(acc, xq[:, perm].astype(np.int32))


def test_one_hot_activation_reads_a_column():
    rng = np.random.default_rng(4)
    M, K = 48, 512
    w = _rand_w(rng, M, K)
    x = np.zeros((1, K), np.float32)
    x[0, 301] = -2.5
    out = oracle.forward(oracle.pack(w, 0.5)[0], M, K, x)
    assert out["xq"][0, 301] == -127
    np.testing.assert_array_equal(out["acc"][0], -127 * w[:, 301].astype(np.int32))


def test_selected_rows_match_full_product():
    rng = np.random.default_rng(12)
    M, K, N = 64, 512, 2
    w = _rand_w(rng, M, K)
    p, _ = oracle.pack(w, 1.0)
    xq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    full = oracle.matmul_i32(p, M, K, xq)
    rows = np.array([63, 0, 17, 17, 40])
    np.testing.assert_array_equal(oracle.matmul_i32(p, M, K, xq, rows), full[:, rows])


def test_int32_range_at_largest_supported_k():
    # |acc| <= 127*K; the largest K with 127*K < 2^24 and K % 256 == 0 is
    # 131840, so the float conversion of the sum is still exact.
    K = 131840
    M = 16
    xq = np.full((1, K), 127, np.int8)
    acc = oracle.matmul_i32(oracle.pack(np.ones((M, K), np.int8), 1.0)[0], M, K, xq)
    assert np.all(acc == 127 * K)
    assert 127 * K < 2**24


@pytest.mark.parametrize("M,K,N", [(16, 256, 1), (32, 512, 6), (64, 1024, 9)])
def test_brute_force_against_float64_matmul(M, K, N):
    # The whole path (quantize, integer product, dequantize) against a float64
    # library matmul of the dequantized operands: (s_w * W) @ (s_a/127 * xq)^T.
    rng = np.random.default_rng(M + K + N)
    w = _rand_w(rng, M, K)
    s_w = 0.0275
    x = (rng.standard_normal((N, K)) * 2).astype(np.float32)
    out = oracle.forward(oracle.pack(w, s_w)[0], M, K, x)
    Wd = torch.from_numpy(w.astype(np.float64)) * float(np.float32(s_w))
    Xd = (torch.from_numpy(out["xq"].astype(np.float64))
          * torch.from_numpy(out["x_scale"].astype(np.float64))[:, None] / 127.0)
    ref = (Xd @ Wd.T).numpy()
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    # and the float result approximates the unquantized product
    approx = x.astype(np.float64) @ (w.astype(np.float64) * float(np.float32(s_w))).T
    assert np.abs(out["y"] - approx).max() <= 0.5 * np.abs(x).max() / 127 * s_w * K


def test_zero_token_gives_zero_output():
    rng = np.random.default_rng(1)
    M, K = 16, 256
    w = _rand_w(rng, M, K)
    x = np.zeros((2, K), np.float32)
    x[1] = rng.standard_normal(K)
    out = oracle.forward(oracle.pack(w, 1.0)[0], M, K, x)
    assert np.all(out["y"][0] == 0) and out["x_scale"][0] == 0
    assert np.any(out["y"][1] != 0)


def test_empty_batch():
    M, K = 16, 256
    p, _ = oracle.pack(np.zeros((M, K), np.int8), 1.0)
    acc = oracle.matmul_i32(p, M, K, np.zeros((0, K), np.int8))
    assert acc.shape == (0, M)
