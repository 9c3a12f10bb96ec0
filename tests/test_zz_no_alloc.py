"""The allocation-free layer driver (static scratch) against bt_layer_forward
(caller's workspace), through the C ABI: identical int32 sums and identical
bf16 outputs, on consecutive calls whose second input is smaller than the
first (the static scratch keeps the first call's contents)."""
import pytest
import torch

import ternary_weight_quantized_bt_amd as bt
import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
TORCH_DT = {bt.BT_I32: torch.int32, bt.BT_BF16: torch.bfloat16}


def _layer(wl, layer=0):
    ws = W.layer_weights(wl, layer, device=DEV)
    return bt.Layer([bt.pack(w, s) for (w, s) in ws], wl.shapes)


def _both(L, xs, ydt):
    """(bt_layer_forward outputs, bt_layer_forward_noalloc outputs)."""
    N = xs[0].shape[0]
    ref = L.forward(xs, y_dtype=ydt)
    ys = L.alloc_outputs(N, ydt, DEV)
    for y in ys:  # a value the kernels must overwrite
        y.view(torch.uint8).fill_(0x5A)
    io = L.make_io(xs, ys, ydt, None)
    bt.bt_layer_forward_noalloc(L.c, io)
    torch.cuda.synchronize()
    return ref, ys


@pytest.mark.parametrize("wl,Ns", [
    # prefill (29.9 MB of scratch, near the 32 MiB limit), then the 64-token
    # matrix-core decode and one token (one launch, no scratch)
    (W.LAYER2B_N1, (2048, 64, 1)),
    # the 70B-class block: 8 tokens (matrix-core decode), then 5, then 1
    (W.STREAM70B, (8, 5, 1)),
])
def test_noalloc_equals_workspace_driver(wl, Ns):
    L = _layer(wl)
    for N in Ns:
        print(f"noalloc {wl.name} N={N}", flush=True)
        xs = [x.to(DEV) for x in W.layer_inputs(wl, 0, N)]
        need = L.workspace_bytes(N)
        assert need <= bt.BT_NOALLOC_SCRATCH_BYTES
        for ydt in (bt.BT_I32, bt.BT_BF16):
            ref, got = _both(L, xs, ydt)
            for p in range(bt.BT_LAYER_PROJ):
                assert torch.equal(ref[p], got[p]), (wl.name, N, ydt, p)


def test_noalloc_too_many_tokens_launches_nothing():
    L = _layer(W.LAYER2B_N1)
    N = 4096  # 59.9 MB of scratch
    assert L.workspace_bytes(N) > bt.BT_NOALLOC_SCRATCH_BYTES
    xs = [torch.zeros((N, K), dtype=torch.bfloat16, device=DEV) for K in L.input_widths()]
    ys = L.alloc_outputs(N, bt.BT_I32, DEV)
    for y in ys:
        y.fill_(7)
    io = L.make_io(xs, ys, bt.BT_I32, None)
    with pytest.raises(bt.BtError) as e:
        bt.bt_layer_forward_noalloc(L.c, io)
    assert e.value.status == bt.BT_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert all(bool((y == 7).all()) for y in ys)
