"""The layer driver captured in a HIP graph: every replay, with eager work and
synchronizations between replays, equals the eager result.  (No kernel of the
library records a memset, so the step is capturable.)"""
import pytest
import torch

import ternary_weight_quantized_bt_amd as bt
import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


@pytest.mark.parametrize("N", [1, 8, 200])
def test_graph_replays_match_eager(N):
    wl = W.LAYER2B_N1
    layers = []
    for l in range(2):
        packed = [bt.pack(w.to(DEV), s) for w, s in W.layer_weights(wl, l)]
        layers.append(bt.Layer(packed, wl.shapes))
    xs = [[x.to(DEV) for x in W.layer_inputs(wl, l, N)] for l in range(2)]
    ws = layers[0].alloc_workspace(N, DEV)
    ys = [L.alloc_outputs(N, bt.BT_BF16, DEV) for L in layers]
    ios = [L.make_io(x, y, bt.BT_BF16, ws) for L, x, y in zip(layers, xs, ys)]

    def step():
        for L, io in zip(layers, ios):
            bt.bt_layer_forward(L.c, io)

    step()
    torch.cuda.synchronize()
    eager = [[y.clone() for y in yl] for yl in ys]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for yl in ys:
            for y in yl:
                y.fill_(0)           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for yl, el in zip(ys, eager):
            for y, e in zip(yl, el):
                assert torch.equal(y, e), f"replay {rep} differs"
        step()                       # eager launch between replays
        torch.cuda.synchronize()


def test_weight_quantizer_graph_replays():
    # the state block is cleared by a fill kernel, so replays start clean
    M, K = 64, 1024
    ws_bytes = bt.bt_quantize_weights_workspace_bytes()
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    w = W.float_weights(M, K, "wide", 3).to(DEV)
    packed = torch.empty(bt.bt_packed_bytes(M, K), dtype=torch.uint8, device=DEV)
    stats = torch.empty(2, dtype=torch.float32, device=DEV)

    def step():
        bt.bt_quantize_weights(w, bt.BT_F32, M, K, bt.BT_WSCALE_ABSMEAN, 1e-5, packed,
                               stats, ws, ws_bytes)

    step()
    torch.cuda.synchronize()
    ref_packed, ref_stats = packed.clone(), stats.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        packed.fill_(0)
        stats.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(packed, ref_packed), f"replay {rep} packed"
        assert torch.equal(stats, ref_stats), f"replay {rep} stats"
        step()
        torch.cuda.synchronize()


def test_base3_graph_replays():
    # base-3 packing and decode products (every launch shape of the product:
    # no K split on a tall matrix, a K split on a short one, four tokens)
    # captured together; replays equal the eager results
    shapes = [(24576, 1024), (64, 4096)]
    mats = []
    for i, (M, K) in enumerate(shapes):
        w = W.ternary_weights(M, K, "p0_0.4", 40 + i, device=DEV)
        packed = torch.empty(bt.bt_b3_bytes(M, K), dtype=torch.uint8, device=DEV)
        outs = []
        for N in (1, 4):
            xq, xs, xsum = bt.quant_act(W.activations(N, K, "normal", 50 + i + N, "bf16",
                                                      device=DEV))
            outs.append((N, xq, xs, xsum, torch.empty((N, M), dtype=torch.bfloat16, device=DEV)))
        mats.append((M, K, w, packed, outs))

    def step():
        for M, K, w, packed, outs in mats:
            bt.bt_pack_ternary_b3(w, M, K, 0.02, packed)
            for N, xq, xs, xsum, y in outs:
                bt.bt_ternary_gemv_b3(packed, M, K, xq, xs, xsum, N, y, bt.BT_BF16)

    step()
    torch.cuda.synchronize()
    eager = [(m[3].clone(), [o[4].clone() for o in m[4]]) for m in mats]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for m in mats:
            m[3].fill_(0)
            for o in m[4]:
                o[4].fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m, (ep, ey) in zip(mats, eager):
            assert torch.equal(m[3], ep), f"replay {rep} packed"
            for o, e in zip(m[4], ey):
                assert torch.equal(o[4], e), f"replay {rep} N={o[0]}"
        step()
        torch.cuda.synchronize()
