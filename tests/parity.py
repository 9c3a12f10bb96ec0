"""Comparison helpers for the GPU parity tests (GPU result vs oracle)."""
import numpy as np
import torch

import oracle
import ternary_weight_quantized_bt_amd as bt

# Float tolerances: relative error of the dequantized output.
RTOL = {bt.BT_F32: 1e-6, bt.BT_BF16: 1e-2}


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).numpy()
    return t.numpy()


def x_for_oracle(x: torch.Tensor) -> np.ndarray:
    """float32 array, or bfloat16 bit patterns as uint16."""
    return to_np(x)


def as_f64(y: torch.Tensor) -> np.ndarray:
    return y.detach().float().cpu().numpy().astype(np.float64)


def assert_rel_close(y: np.ndarray, ref: np.ndarray, rtol: float, what=""):
    assert y.shape == ref.shape, (y.shape, ref.shape)
    err = np.abs(y - ref)
    bad = err > rtol * np.abs(ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outputs off; first at {tuple(i)}: "
            f"got {y[tuple(i)]!r}, oracle {ref[tuple(i)]!r}, rel {err[tuple(i)] / max(abs(ref[tuple(i)]), 1e-300):.3g}")


def assert_equal(a: np.ndarray, b: np.ndarray, what=""):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if not np.array_equal(a, b):
        d = np.argwhere(a != b)
        raise AssertionError(f"{what}: {len(d)} of {a.size} differ; first at "
                             f"{tuple(d[0])}: {a[tuple(d[0])]} vs {b[tuple(d[0])]}")


def check_projection(packed_gpu, packed_ref, M, K, xq_ref, xs_ref, acc_ref_rows,
                     y_gpu, ydt, rows=None, what=""):
    """Compare a GPU output [N, M] (or its selected rows) with the oracle."""
    y = y_gpu if rows is None else y_gpu[:, torch.as_tensor(rows, device=y_gpu.device)]
    if ydt == bt.BT_I32:
        assert_equal(to_np(y), acc_ref_rows, what)
    else:
        ref = oracle.dequant(acc_ref_rows, oracle.scale_of(packed_ref, M, K), xs_ref)
        assert_rel_close(as_f64(y), ref, RTOL[ydt], what)


# ------------------------------------------------------------ canaries ----

GUARD = 4096      # sentinel bytes before and after each guarded output
SENTINEL = 0xA5

_ELEM = {torch.int8: 1, torch.uint8: 1, torch.bfloat16: 2, torch.int16: 2,
         torch.float32: 4, torch.int32: 4}


class Guarded:
    """An output tensor with GUARD sentinel bytes on each side, in one
    allocation (the output itself starts 16-byte aligned and filled with the
    sentinel): a kernel that writes past either end of its output changes a
    sentinel byte, which check() reports."""

    def __init__(self, shape, dtype, device="cuda:0"):
        n = int(np.prod(shape)) * _ELEM[dtype]
        self.n = n
        self.buf = torch.full((2 * GUARD + (n + 15) // 16 * 16,), SENTINEL,
                              dtype=torch.uint8, device=device)
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(*shape)

    def check(self, what=""):
        b = self.buf.cpu().numpy()
        front, back = b[:GUARD], b[GUARD + self.n:]
        for name, band in (("before", front), ("after", back)):
            bad = np.flatnonzero(band != SENTINEL)
            if bad.size:
                raise AssertionError(f"{what}: {bad.size} sentinel bytes {name} the output "
                                     f"changed (first at band offset {bad[0]})")


def guarded(shape, dtype, device="cuda:0"):
    """A Guarded output and its tensor."""
    g = Guarded(shape, dtype, device)
    return g, g.t
