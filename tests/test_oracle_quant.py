"""Pins of the oracle's per-token absmax int8 quantization."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

import oracle
from conftest import read_golden


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (test helper)."""
    u = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@pytest.mark.parametrize("row", read_golden("quant_worked_examples.txt"),
                         ids=lambda r: r[0])
def test_worked_examples(row):
    name, xs, scale, codes, total = row
    x = np.array([[float(v) for v in xs.split()]], np.float32)
    xq, s, sm = oracle.quant_act(x)
    assert xq[0].tolist() == [int(v) for v in codes.split()]
    assert s[0] == np.float32(float(scale))
    assert sm[0] == int(total)


def test_outlier_row_crushes_normal_features():
    # The outlier figure's point: everything but the outlier becomes 0.
    x = np.array([[0.04, -0.11, 48.72, 0.02, -0.15, 0.08]], np.float32)
    xq, _, _ = oracle.quant_act(x)
    assert np.count_nonzero(xq) == 1


finite = st.floats(-1e6, 1e6, allow_nan=False, allow_infinity=False, width=32)


@settings(max_examples=200, deadline=None)
@given(hnp.arrays(np.float32, st.tuples(st.integers(1, 3), st.integers(1, 300)),
                  elements=finite))
def test_invariants(x):
    xq, s, sm = oracle.quant_act(x)
    for n in range(x.shape[0]):
        amax = np.abs(x[n]).max()
        assert s[n] == amax
        if amax == 0 or amax < 1e-30:
            if amax == 0:
                assert np.all(xq[n] == 0)
            continue
        # the largest magnitude maps to +-127
        assert np.abs(xq[n].astype(int)).max() == 127
        # sign is kept or the value becomes 0
        assert np.all((xq[n] == 0) | (np.sign(xq[n]) == np.sign(x[n])))
        # within half a step (plus binary32 slack) of the exact scaled value
        exact = x[n].astype(np.float64) * 127.0 / float(amax)
        assert np.all(np.abs(xq[n] - exact) <= 0.5 + 1e-4)
        assert sm[n] == int(xq[n].astype(np.int64).sum())


def test_bf16_input_matches_its_widened_float32():
    rng = np.random.default_rng(3)
    x32 = rng.standard_normal((5, 512)).astype(np.float32) * 3
    bits = _bf16_bits(x32)
    widened = (bits.astype(np.uint32) << 16).view(np.float32)
    a = oracle.quant_act(bits)
    b = oracle.quant_act(widened)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_scale_invariance_by_powers_of_two():
    # x and 2^e * x quantize to the same codes (both amax and every product
    # scale exactly by 2^e in binary32).
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 1000)).astype(np.float32)
    a = oracle.quant_act(x)
    b = oracle.quant_act(x * np.float32(8.0))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1] * 8, b[1])


def test_subnormals_quantize_to_zero_without_amax_change():
    x = np.array([[1.0, 1e-40, -1e-42, 0.0]], np.float32)
    xq, s, _ = oracle.quant_act(x)
    assert xq[0].tolist() == [127, 0, 0, 0]
    assert s[0] == 1.0


def test_overflowing_reciprocal_keeps_binary32_steps():
    # amax below 127 / FLT_MAX: 127 / amax is +inf in binary32, so x * inv is
    # +-inf for every nonzero x and the clamp gives 127 * sign(x); 0 * inf is
    # taken as 0.  Whether amax is normal or subnormal.  This is not the real
    # value of x * 127 / amax: 2e-38 * 127 / 1e-37 = 25.4 (row 0, column 3)
    # still gets 127.
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(127.0) / np.float32(1e-37))
    x = np.array([[1e-37, -5e-38, 0.0, 2e-38, -0.0],
                  [0.0, 1e-40, -3e-40, 2e-41, 0.0]], np.float32)
    xq, s, sm = oracle.quant_act(x)
    assert xq[0].tolist() == [127, -127, 0, 127, 0]
    assert xq[1].tolist() == [0, 127, -127, 127, 0]
    assert sm.tolist() == [127, 127]
    assert s[0] == np.float32(1e-37) and s[1] == np.float32(3e-40)
