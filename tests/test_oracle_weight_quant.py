"""Pins of the oracle's float -> ternary weight quantizer (AbsMean / max|w|,
RoundClip): hand-worked examples, exact rational arithmetic, closed forms
and properties that follow from the definitions."""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

import oracle
from conftest import read_golden
from oracle import weight_quant as wq


def _f(x) -> Fraction:
    return Fraction(float(x))


def _is_nearest_f32(r: np.float32, v: Fraction) -> bool:
    """r is the float32 nearest to v >= 0, ties to an even significand."""
    r = np.float32(r)
    lo = np.nextafter(r, np.float32(0))
    hi = np.nextafter(r, np.float32(np.inf))
    dr = abs(_f(r) - v)
    for nb in (lo, hi):
        if nb == r or not np.isfinite(nb):
            continue
        dn = abs(_f(nb) - v)
        if dn < dr:
            return False
        if dn == dr and (int(np.float32(r).view(np.uint32)) & 1):
            return False
    return True


@pytest.mark.parametrize("row", read_golden("weight_quant_examples.txt"),
                         ids=lambda r: r[0])
def test_worked_examples(row):
    name, mode, eps, ws, s, d, codes = row
    w = np.array([float(v) for v in ws.split()], np.float32)
    got, gs, gd = wq.ternarize(w, mode, float(eps))
    assert got.tolist() == [int(c) for c in codes.split()]
    assert gs == np.float32(float(s))
    assert gd == np.float32(float(d))


def test_round_clip_definition_table():
    # RoundClip(x, -1, 1) = max(-1, min(1, round(x))), half to even
    q = np.array([-7.0, -1.5, -1.0, -0.5000001, -0.5, -0.4999999, -0.0, 0.0,
                  0.25, 0.5, 0.50000006, 0.9, 1.5, 2.5, np.inf, -np.inf, np.nan],
                 np.float32)
    want = [-1, -1, -1, -1, 0, 0, 0, 0, 0, 0, 1, 1, 1, 1, 1, -1, 0]
    assert wq.round_clip(q).tolist() == want


# ---- round_ratio_f32: the one rounding of the exact mean --------------------

def test_round_ratio_hand_cases():
    # exact values
    assert wq.round_ratio_f32(3, 4) == np.float32(0.75)
    assert wq.round_ratio_f32(1, 1) == np.float32(1.0)
    # 1 + 2**-24 lies halfway between 1 and 1 + 2**-23: even -> 1
    assert wq.round_ratio_f32(2**24 + 1, 2**24) == np.float32(1.0)
    # 1 + 3 * 2**-24 lies halfway between 1 + 2**-23 and 1 + 2**-22: even
    assert wq.round_ratio_f32(2**24 + 3, 2**24) == np.float32(1 + 2.0**-22)
    # just above a halfway point rounds up
    assert wq.round_ratio_f32(2**25 + 3, 2**25) == np.float32(1 + 2.0**-23)
    # subnormal quantum 2**-149: 2**-150 is halfway to 0 (even -> 0),
    # 3 * 2**-150 is halfway between 2**-149 and 2**-148 (even -> 2**-148)
    assert wq.round_ratio_f32(1, 2**150) == np.float32(0.0)
    assert wq.round_ratio_f32(3, 2**150) == np.float32(2.0**-148)
    assert wq.round_ratio_f32(5, 2**151) == np.float32(2.0**-149)  # 1.25 quanta
    # the largest finite float32 stays finite
    fmax = np.finfo(np.float32).max
    num = int(Fraction(float(fmax)))
    assert wq.round_ratio_f32(num * 7, 7) == fmax


@settings(max_examples=400, deadline=None)
@given(st.integers(1, 2**200), st.integers(1, 2**200), st.integers(-180, 100))
def test_round_ratio_is_nearest(a, b, sh):
    num, den = (a << sh, b) if sh >= 0 else (a, b << -sh)
    v = Fraction(num, den)
    if v > _f(np.finfo(np.float32).max):
        return
    assert _is_nearest_f32(wq.round_ratio_f32(num, den), v)


# ---- the statistic -----------------------------------------------------------

@settings(max_examples=150, deadline=None)
@given(hnp.arrays(np.float32, st.integers(1, 64),
                  elements=st.floats(-2.0**100, 2.0**100, allow_nan=False, width=32)))
def test_abs_mean_is_the_rounded_exact_mean(w):
    # brute force with exact fractions
    v = sum((abs(_f(x)) for x in w), Fraction(0)) / w.size
    g = wq.abs_mean(w)
    assert _is_nearest_f32(g, v)


def test_abs_mean_does_not_depend_on_summation_order():
    # one large value and many tiny ones: a float32 running sum drops every
    # tiny term, the exact mean keeps them
    n = 4096
    w = np.full(n, 2.0**-24, np.float32)
    w[0] = 1.0
    exact = (Fraction(1) + (n - 1) * Fraction(1, 2**24)) / n
    g = wq.abs_mean(w)
    assert _is_nearest_f32(g, exact)
    naive = np.float32(0)
    for x in w:
        naive = np.float32(naive + x)
    assert np.float32(naive / np.float32(n)) != g
    assert wq.abs_mean(w[::-1].copy()) == g


def test_abs_mean_closed_forms():
    rng = np.random.default_rng(5)
    # constant magnitude c: mean |W| = c exactly
    c = np.float32(0.0371)
    w = (c * rng.choice([-1, 1], size=(32, 256))).astype(np.float32)
    assert wq.abs_mean(w) == c
    # a pre-ternarized tensor {-g, 0, +g} with half its entries nonzero:
    # mean = g / 2 exactly (g a power of two)
    t = rng.choice([-1, 1], size=(32, 256)).astype(np.float32)
    t[:, ::2] = 0
    assert wq.abs_mean(np.float32(2.0**-5) * t) == np.float32(2.0**-6)
    # subnormal weights: mean of {2**-149, 0} = 2**-150, halfway -> 0 (even)
    assert wq.abs_mean(np.array([2.0**-149, 0.0], np.float32)) == 0
    assert wq.abs_mean(np.array([2.0**-149, 2.0**-148], np.float32)) == np.float32(2.0**-148)


def test_bf16_bits_are_widened_exactly():
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 2**16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    w32 = (bits.astype(np.uint32) << 16).view(np.float32)
    assert wq.abs_mean(bits) == wq.abs_mean(w32)
    assert wq.abs_max(bits) == wq.abs_max(w32)


# ---- ternarization -----------------------------------------------------------

@settings(max_examples=150, deadline=None)
@given(hnp.arrays(np.float32, st.integers(1, 200),
                  elements=st.floats(-1e4, 1e4, allow_nan=False, width=32)),
       st.sampled_from([wq.ABSMEAN, wq.ABSMAX]),
       st.sampled_from([0.0, 1e-5, 0.01, 3.0]))
def test_codes_follow_the_exact_ratio(w, mode, eps):
    # float32 division is correctly rounded and rounding is monotone, so
    # round(float32(w / d)) is +-1 exactly when |w| / d exceeds the midpoint
    # between 0.5 and the next float32 up, 0.5 + 2**-25
    codes, s, d = wq.ternarize(w, mode, eps)
    assert d == np.float32(s + np.float32(eps))
    for x, c in zip(w, codes):
        if d == 0:
            want = int(np.sign(x))
        else:
            want = int(np.sign(x)) if abs(_f(x)) / _f(d) > Fraction(1, 2) + Fraction(1, 2**25) else 0
        assert c == want, (x, d)


def test_pre_ternarized_weights_come_back_exactly():
    # [I2S]'s max|w| scale on a tensor already rounded to {-g, 0, +g}
    rng = np.random.default_rng(11)
    t = rng.choice([-1, 0, 1], size=(48, 512), p=[0.3, 0.4, 0.3]).astype(np.int8)
    g = np.float32(0.0213)
    w = (g * t).astype(np.float32)
    codes, s, d = wq.ternarize(w, wq.ABSMAX, 0.0)
    assert s == g and d == g
    assert np.array_equal(codes, t)
    # and the AbsMean scale (about 0.6 g) maps +-g to +-1.67 -> clipped +-1
    codes2, s2, _ = wq.ternarize(w, wq.ABSMEAN, 0.0)
    assert np.array_equal(codes2, t)
    assert abs(float(s2) - 0.6 * float(g)) < 0.05 * float(g)


def test_packed_result_round_trips():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((32, 512)) * 0.02).astype(np.float32)
    packed, s, d = wq.quantize_weights(w, wq.ABSMEAN, 1e-5)
    codes, s2, d2 = wq.ternarize(w, wq.ABSMEAN, 1e-5)
    assert np.array_equal(oracle.unpack(packed, 32, 512), codes)
    assert oracle.scale_of(packed, 32, 512) == d == d2
    # about 68% of a normal's mass lies beyond gamma/2 ~ 0.4 sigma
    assert 0.6 < np.count_nonzero(codes) / codes.size < 0.75


def test_bad_arguments():
    w = np.ones(4, np.float32)
    with pytest.raises(ValueError):
        wq.ternarize(w, wq.ABSMEAN, -1e-5)
    with pytest.raises(ValueError):
        wq.ternarize(w, wq.ABSMEAN, float("nan"))
    with pytest.raises(ValueError):
        wq.ternarize(w, "absmedian", 0.0)
    with pytest.raises(TypeError):
        wq.ternarize(w.astype(np.float64), wq.ABSMEAN, 0.0)
