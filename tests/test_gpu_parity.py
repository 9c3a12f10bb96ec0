"""GPU path vs CPU oracle on seeded inputs: exact packed bytes, int8 codes,
scales, sums and int32 products; float outputs within 1e-6 (fp32) or 1e-2
(bf16) relative.  Shapes span several tiles and ragged tails in every
dimension the kernels tile (tokens, row tiles per workgroup, K blocks per
wave)."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt
import workloads as W
from parity import (RTOL, as_f64, assert_equal, assert_rel_close,
                    check_projection, to_np, x_for_oracle)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _w(M, K, seed, dist="p0_0.4"):
    return W.ternary_weights(M, K, dist, seed)


def _x(N, K, seed, dtype="f32", dist="normal", frac=0.0, scale=1.0):
    return W.activations(N, K, dist, seed, dtype, frac, scale)


# ------------------------------------------------------------------ pack ----

@pytest.mark.parametrize("M,K", [(16, 256), (48, 768), (80, 2304), (640, 2560),
                                 (2560, 6912)])
def test_pack_bytes_exact(M, K):
    w = _w(M, K, M + K, "uniform")
    ref, bad = oracle.pack(w.numpy(), 0.0275)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    packed = bt.pack(w.to(DEV), 0.0275, invalid_count=cnt)
    assert_equal(to_np(packed), ref, "packed bytes")
    assert int(cnt.item()) == bad == 0
    back = bt.unpack(packed, M, K)
    assert_equal(to_np(back), w.numpy(), "unpack round trip")


def test_pack_invalid_values_clamped_and_counted():
    M, K = 32, 512
    w = _w(M, K, 5, "uniform")
    w[0, 0] = 7
    w[5, 300] = -128
    w[31, 511] = 2
    w[17, 17] = -2
    ref, bad = oracle.pack(w.numpy(), 1.0)
    cnt = torch.full((1,), 3, dtype=torch.int32, device=DEV)  # kernel adds
    packed = bt.pack(w.to(DEV), 1.0, invalid_count=cnt)
    assert_equal(to_np(packed), ref, "packed bytes")
    assert bad == 4 and int(cnt.item()) == 3 + 4


# ----------------------------------------------------------------- quant ----

@pytest.mark.parametrize("N,K,dtype,dist,frac,scale", [
    (1, 2560, "f32", "normal", 0.0, 1.0),
    (3, 256, "f32", "normal", 0.0, 1.0),
    (64, 6912, "bf16", "normal", 0.01, 20.0),
    (2048, 2560, "bf16", "student_t4", 0.0, 1.0),
    (8, 28672, "bf16", "normal", 0.005, 30.0),
    (2, 131840, "f32", "normal", 0.0, 1.0),
])
def test_quant_exact(N, K, dtype, dist, frac, scale):
    x = _x(N, K, N * 7 + K, dtype, dist, frac, scale)
    xq, xs, xsum = bt.quant_act(x.to(DEV))
    rq, rs, rsum = oracle.quant_act(x_for_oracle(x))
    assert_equal(to_np(xq), rq, "xq")
    assert_equal(to_np(xs), rs, "scale")
    assert_equal(to_np(xsum), rsum, "sum")


def double_rounding_row(K, amax=100.0):
    """A row with max |x| = amax whose other values x make the binary32
    product x * fl(127 / amax) land exactly on a half-integer while the exact
    product does not: rounding the rounded product (the contract) and
    rounding the exact product (a fused multiply-add) give different codes."""
    amax = np.float32(amax)
    inv = np.float32(np.float32(127.0) / amax)
    row = np.zeros(K, np.float32)
    row[0] = amax
    n = 1
    for k in range(-126, 127):
        t = k + 0.5
        x0 = np.float32(t / float(inv))
        for x in (np.nextafter(x0, np.float32(-1e9)), x0, np.nextafter(x0, np.float32(1e9))):
            p64 = float(x) * float(inv)
            if (float(np.float32(p64)) == t and p64 != t and abs(x) < amax and n < K
                    and np.floor(p64 + 0.5) != np.rint(np.float32(p64))):
                row[n] = x
                n += 1
    assert n > 64
    return torch.from_numpy(row)


def test_quant_special_rows():
    K = 512
    x = torch.zeros((9, K), dtype=torch.float32)
    x[1, 3] = -2.5                       # single negative max
    x[2] = torch.linspace(-127, 127, K)  # ties at exact .5 after scaling by 1
    x[2, 0] = -127.0
    x[3, :5] = torch.tensor([127.0, 2.5, -2.5, 3.5, 0.5])
    x[4] = 1e-40                         # subnormals only
    x[4, 9] = 1.0
    x[5, 100] = 48.72                    # the outlier row of the worked example
    x[5, :6] = torch.tensor([0.04, -0.11, 48.72, 0.02, -0.15, 0.08])
    x[6, :4] = torch.tensor([1e-37, -5e-38, 0.0, 2e-38])  # 127/amax overflows
    x[7, 10:13] = torch.tensor([1e-40, -3e-40, 2e-41])     # subnormal amax
    x[8] = double_rounding_row(K)                          # product rounds before rint
    xq, xs, xsum = bt.quant_act(x.to(DEV))
    rq, rs, rsum = oracle.quant_act(x.numpy())
    assert_equal(to_np(xq), rq, "xq")
    assert_equal(to_np(xs), rs, "scale")
    assert_equal(to_np(xsum), rsum, "sum")
    assert to_np(xs)[0] == 0 and not to_np(xq)[0].any()


# --------------------------------------------------------------- matmul ----

SHAPES = [(16, 256), (48, 768), (80, 1280), (208, 2304), (1024, 2560)]
NS = [1, 2, 3, 4, 5, 8, 16, 17, 63, 64, 65, 130, 257]


def _case(M, K, N, seed):
    w = _w(M, K, seed)
    x = _x(N, K, seed + 1, "bf16", "normal", 0.01, 20.0)
    ref_packed, _ = oracle.pack(w.numpy(), 0.02 + (seed % 7) * 0.001)
    ref = oracle.forward(ref_packed, M, K, x_for_oracle(x))
    packed = bt.pack(w.to(DEV), 0.02 + (seed % 7) * 0.001)
    xq, xs, xsum = bt.quant_act(x.to(DEV))
    return ref_packed, ref, packed, xq, xs, xsum


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
@pytest.mark.parametrize("M,K", SHAPES)
def test_matmul_int32_exact(fn, M, K):
    for N in NS:
        ref_packed, ref, packed, xq, xs, xsum = _case(M, K, N, M * 31 + K + N)
        y = getattr(bt, fn)(packed, M, K, xq, xs, xsum, bt.BT_I32)
        assert_equal(to_np(y), ref["acc"], f"{fn} M={M} K={K} N={N}")


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
@pytest.mark.parametrize("ydt", [bt.BT_F32, bt.BT_BF16])
def test_matmul_float_within_tolerance(fn, ydt):
    for (M, K) in SHAPES[:4]:
        for N in (1, 3, 17, 64, 130):
            ref_packed, ref, packed, xq, xs, xsum = _case(M, K, N, M + K * 3 + N)
            y = getattr(bt, fn)(packed, M, K, xq, xs, xsum, ydt)
            assert_rel_close(as_f64(y), ref["y"], RTOL[ydt], f"{fn} {M}x{K} N={N}")


@pytest.mark.parametrize("M,K,N", [
    (48, 10240, 16),    # 16 rows x 10240 columns: too long for LDS, B from global memory
    (80, 16384, 9),     # 9 rows x 16 KiB: global B, ragged token group
    (48, 10240, 20),    # two token groups, the second ragged, global B
    (112, 8192, 8),     # 8 rows x 8 KiB: staged in LDS, two workgroups per CU
    (48, 8448, 16),     # 16 rows x 8448: staged, one workgroup per CU
    (32, 768, 33),      # three token groups, one token in the last
])
def test_batched_decode_staging_modes(M, K, N):
    """Both B sources of the batched-decode kernel (codes staged in LDS, or
    read from global memory when the rows are too long), ragged token groups."""
    ref_packed, ref, packed, xq, xs, xsum = _case(M, K, N, 7 * M + K + N)
    for ydt in (bt.BT_I32, bt.BT_F32, bt.BT_BF16):
        y = bt.gemv(packed, M, K, xq, xs, xsum, ydt)
        if ydt == bt.BT_I32:
            assert_equal(to_np(y), ref["acc"], f"M={M} K={K} N={N}")
        else:
            assert_rel_close(as_f64(y), ref["y"], RTOL[ydt], f"M={M} K={K} N={N} ydt={ydt}")


@pytest.mark.parametrize("M,K,N", [
    (4096, 2304, 2),    # tall group, 2 tokens: dot4
    (4096, 2304, 3),    # tall group, 3 tokens: matrix cores
    (4112, 2304, 4),    # tall, odd tile count, 4 tokens: matrix cores
    (4096, 16640, 2),   # tall with long rows, 2 tokens: matrix cores
    (48, 16640, 2),     # short group with long rows, 2 tokens: dot4
    (64, 17408, 3),     # codes of 4 token slots beyond the dot4 kernel's LDS: matrix cores
])
def test_decode_kernel_choice_few_tokens(M, K, N):
    """2..4 tokens run on the dot4 kernel or on the matrix cores depending on
    the group's shape; either way exact in int32 against the oracle, and
    equal bit for bit to the prefill kernel."""
    ref_packed, ref, packed, xq, xs, xsum = _case(M, K, N, 3 * M + K + N)
    for ydt in (bt.BT_I32, bt.BT_BF16):
        y = bt.gemv(packed, M, K, xq, xs, xsum, ydt)
        assert torch.equal(y, bt.gemm(packed, M, K, xq, xs, xsum, ydt)), (M, K, N, ydt)
        if ydt == bt.BT_I32:
            assert_equal(to_np(y), ref["acc"], f"M={M} K={K} N={N}")
        else:
            assert_rel_close(as_f64(y), ref["y"], RTOL[ydt], f"M={M} K={K} N={N}")


def test_batched_decode_three_k_phases_sampled():
    """Rows too long for LDS (12 tokens x 25600 columns): three K phases with
    int32 partial sums carried in LDS, several tiles per workgroup, a ragged
    last phase; sampled output rows against the oracle."""
    M, K, N = 9600, 25600, 12
    w = _w(M, K, 5150)
    x = _x(N, K, 5151, "bf16", "normal", 0.005, 30.0)
    ref_packed, _ = oracle.pack(w.numpy(), 0.02)
    xq_ref, xs_ref, _ = oracle.quant_act(x_for_oracle(x))
    packed = bt.pack(w.to(DEV), 0.02)
    xq, xs, xsum = bt.quant_act(x.to(DEV))
    rows = np.sort(np.random.default_rng(7).choice(M, 96, replace=False))
    acc = oracle.matmul_i32(ref_packed, M, K, xq_ref, rows)
    y = to_np(bt.gemv(packed, M, K, xq, xs, xsum, bt.BT_I32))
    assert_equal(y[:, rows], acc, "three phases")


@pytest.mark.parametrize("M,K,Ns", [
    (208, 2304, (1, 4, 5, 64, 257)),
    # 35 row tiles: two workgroup tiles of 256 whole rows (bf16 results leave
    # through LDS) and a partial one (direct stores); ragged token tiles
    (560, 1024, (128, 130, 200, 257)),
])
def test_gemv_and_gemm_agree_bitwise(M, K, Ns):
    for N in Ns:
        _, _, packed, xq, xs, xsum = _case(M, K, N, 99 + N)
        for ydt in (bt.BT_F32, bt.BT_BF16, bt.BT_I32):
            a = bt.gemv(packed, M, K, xq, xs, xsum, ydt)
            b = bt.gemm(packed, M, K, xq, xs, xsum, ydt)
            assert torch.equal(a, b), (N, ydt)


def test_prefill_persistent_workgroups_take_several_tiles():
    # 16 x 33 = 528 workgroup tiles, more than the resident workgroups, so
    # the persistent grid gives some of them two tiles (and a ragged last
    # token tile); every output against the oracle's int32 sums, bf16 too
    M, K, N = 4096, 512, 2049
    ref_packed, ref, packed, xq, xs, xsum = _case(M, K, N, 777)
    y = bt.gemm(packed, M, K, xq, xs, xsum, bt.BT_I32)
    assert_equal(to_np(y), ref["acc"], "persistent prefill")
    yb = bt.gemm(packed, M, K, xq, xs, xsum, bt.BT_BF16)
    assert_rel_close(as_f64(yb), ref["y"], RTOL[bt.BT_BF16], "persistent prefill bf16")


def test_prefill_bf16_whole_tiles_against_oracle():
    M, K, N = 560, 1024, 200
    ref_packed, ref, packed, xq, xs, xsum = _case(M, K, N, 4242)
    y = bt.gemm(packed, M, K, xq, xs, xsum, bt.BT_BF16)
    assert_rel_close(as_f64(y), ref["y"], RTOL[bt.BT_BF16], "prefill bf16")


def test_special_weights_and_zero_tokens():
    M, K, N = 32, 512, 6
    x = _x(N, K, 3)
    x[2] = 0.0
    xq, xs, xsum = bt.quant_act(x.to(DEV))
    for value in (-1, 0, 1):
        w = torch.full((M, K), value, dtype=torch.int8)
        packed = bt.pack(w.to(DEV), 0.5)
        for fn in (bt.gemv, bt.gemm):
            acc = to_np(fn(packed, M, K, xq, xs, xsum, bt.BT_I32))
            expect = value * to_np(xsum).astype(np.int64)
            assert_equal(acc, np.repeat(expect[:, None], M, 1).astype(np.int32), "constant W")
            y = to_np(fn(packed, M, K, xq, xs, xsum, bt.BT_F32))
            assert not y[2].any()


def test_largest_k_exact():
    # |acc| = 127*K just below 2^24 at K = 131840
    M, K = 16, 131840
    w = torch.ones((M, K), dtype=torch.int8)
    w[3] = -1
    x = torch.ones((2, K), dtype=torch.float32)
    x[1] *= -0.5
    packed = bt.pack(w.to(DEV), 1.0)
    xq, xs, xsum = bt.quant_act(x.to(DEV))
    ref_packed, _ = oracle.pack(w.numpy(), 1.0)
    ref = oracle.forward(ref_packed, M, K, x.numpy())
    for fn in (bt.gemv, bt.gemm):
        acc = to_np(fn(packed, M, K, xq, xs, xsum, bt.BT_I32))
        assert_equal(acc, ref["acc"], "max K")
        assert abs(int(acc[0, 0])) == 127 * K
        y = as_f64(fn(packed, M, K, xq, xs, xsum, bt.BT_F32))
        assert_rel_close(y, ref["y"], 1e-6, "max K float")


def test_largest_n_sampled_tokens():
    """BT_MAX_N tokens of a 256-wide bf16 input (1 GiB) through quant_act and
    both products: exact codes, scales, sums and int32 sums on sampled tokens
    (the first and last 16 and 48 random ones), computed by the oracle from
    those tokens' rows alone (quantization is per token)."""
    N, M, K = bt.BT_MAX_N, 32, 256
    print(f"largest N: N={N} M={M} K={K}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(2 ** 21 + 7)
    x = torch.randn((N, K), generator=g, device=DEV).to(torch.bfloat16)
    w = _w(M, K, 2121)
    packed = bt.pack(w.to(DEV), 0.0125)
    ref_packed, _ = oracle.pack(w.numpy(), 0.0125)
    xq, xs, xsum = bt.quant_act(x)
    rng = np.random.default_rng(2121)
    tok = np.unique(np.r_[np.arange(16), np.arange(N - 16, N), rng.choice(N, 48, replace=False)])
    idx = torch.from_numpy(tok).to(DEV)
    rq, rs, rsum = oracle.quant_act(x_for_oracle(x[idx]))
    assert_equal(to_np(xq[idx]), rq, "codes")
    assert_equal(to_np(xs[idx]), rs, "scales")
    assert_equal(to_np(xsum[idx]), rsum, "code sums")
    acc_ref = oracle.matmul_i32(ref_packed, M, K, rq)
    for fn in (bt.gemv, bt.gemm):
        acc = fn(packed, M, K, xq, xs, xsum, bt.BT_I32)
        assert acc.shape == (N, M)
        assert_equal(to_np(acc[idx]), acc_ref, f"{fn.__name__} int32 at N={N}")
        del acc


def test_empty_batch_with_real_buffers():
    M, K = 16, 256
    packed = bt.pack(torch.zeros((M, K), dtype=torch.int8, device=DEV), 1.0)
    xq = torch.empty((0, K), dtype=torch.int8, device=DEV)
    xs = torch.empty(0, device=DEV)
    xsum = torch.empty(0, dtype=torch.int32, device=DEV)
    for fn in (bt.gemv, bt.gemm):
        y = fn(packed, M, K, xq, xs, xsum, bt.BT_F32)
        assert y.shape == (0, M)


def test_non_default_stream():
    M, K, N = 208, 2304, 37
    ref_packed, ref, packed, xq, xs, xsum = _case(M, K, N, 4242)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y1 = bt.gemv(packed, M, K, xq, xs, xsum, bt.BT_I32, stream=s)
        y2 = bt.gemm(packed, M, K, xq, xs, xsum, bt.BT_I32, stream=s)
    s.synchronize()
    assert_equal(to_np(y1), ref["acc"], "gemv on side stream")
    assert_equal(to_np(y2), ref["acc"], "gemm on side stream")
