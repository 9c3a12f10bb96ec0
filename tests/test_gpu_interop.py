"""GPU to_float and I2_S conversions vs the oracle: every byte and every
output bit identical."""
import numpy as np
import pytest
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt
import workloads as W
from oracle import interop as io
from parity import assert_equal, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
SHAPES = [(16, 256), (48, 768), (80, 2304), (2560, 6912)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("scale", [0.0213, -0.75, 1 + 3 * 2.0**-8])
def test_dequantize(M, K, scale):
    print(f"dequantize {M}x{K} scale={scale}", flush=True)
    w = W.ternary_weights(M, K, "p0_0.4", M * 7 + K)
    packed = bt.pack(w.to(DEV), scale)
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        got = to_np(bt.dequantize(packed, M, K, dt))
        want = io.to_float(w.numpy(), scale, name)
        if name == "f32":
            got, want = got.view(np.uint32), want.view(np.uint32)
        assert_equal(got, want, f"to_float {name}")


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("block", [4, 16, 64, 128, 256, 4096])
def test_i2s_import_export(M, K, block):
    print(f"i2s {M}x{K} block={block}", flush=True)
    w = W.ternary_weights(M, K, "uniform", M + K + block)
    s = 0.0371
    i2s = io.i2s_pack(w.numpy(), s, block)
    ref_packed, _ = oracle.pack(w.numpy(), s)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    packed = bt.i2s_import(torch.from_numpy(i2s).to(DEV), M, K, block, cnt)
    assert_equal(to_np(packed), ref_packed, "imported packed bytes")
    assert int(cnt.item()) == 0
    back = bt.i2s_export(torch.from_numpy(ref_packed).to(DEV), M, K, block)
    assert_equal(to_np(back), i2s, "exported I2_S bytes")


def test_i2s_whole_tensor_block_and_invalid_codes():
    M, K = 32, 512
    w = W.ternary_weights(M, K, "uniform", 9)
    for block in (M * K, M * K // 4):
        i2s = io.i2s_pack(w.numpy(), 0.5, block)
        i2s[3] |= 0xC0   # one code 3
        i2s[100] = 0xFF  # four code-3 values
        want_w, _, bad = io.i2s_unpack(i2s, M, K, block)
        assert bad == 5
        ref_packed, _ = oracle.pack(want_w, 0.5)
        cnt = torch.full((1,), 2, dtype=torch.int32, device=DEV)  # the kernel adds
        packed = bt.i2s_import(torch.from_numpy(i2s).to(DEV), M, K, block, cnt)
        assert_equal(to_np(packed), ref_packed, "imported packed bytes")
        assert int(cnt.item()) == 2 + 5
