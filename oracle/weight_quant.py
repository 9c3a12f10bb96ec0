"""CPU oracle for the float -> ternary weight quantizer.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite, the
package smoke check and the benchmark's CPU-baseline leg are its only callers.

What it computes, cited by page title and section:
  [PARA] "LLM Quantization Paradigms: FP8, AWQ, EXL2 & BitNet b1.58 in 2026",
         section 5 ("The Mathematics of BitNet b1.58"): the AbsMean
         quantizer.  gamma is the mean of |W| over all n*m entries, and
         W~ = RoundClip(W / (gamma + eps), -1, 1) with
         RoundClip(x, a, b) = max(a, min(b, round(x))).
  [I2S]  "How BitNet's 1-Bit (I2_S) Quantization Works Compared to Standard
         LLM Quantization", "Per-Tensor Scaling Strategy": the I2_S scale is
         max|w| of the tensor, one float per tensor.

Readings (the pages leave these open):
  Q1  The statistic s is exact.  For the mean, the sum of |W| is taken as an
      exact real number over the float32 values of W (bfloat16 inputs are
      widened exactly), divided by the entry count, and rounded ONCE to the
      nearest float32 (ties to even).  The result is then independent of any
      summation order.  For the max, s = max|W|.
  Q2  The divisor is d = float32(s + eps), one float32 addition; d is also
      the scale stored with the packed codes, so that d * W~ approximates W.
  Q3  W / d is one float32 division (correctly rounded); round() rounds
      half to even, the IEEE default; 0 / 0 (an all-zero tensor with
      eps = 0) gives code 0.  A nonzero w over d = 0 is +-inf and clips to
      +-1.
  Q4  eps is supplied by the caller: finite and >= 0.
Non-finite weights are outside the contract.
"""
from __future__ import annotations

import numpy as np

ABSMEAN = "absmean"
ABSMAX = "absmax"


def as_f32(w: np.ndarray) -> np.ndarray:
    """float32 values of w: float32 as is, bfloat16 bit patterns (uint16)
    widened exactly (the 16 bits become the high half of a float32)."""
    w = np.asarray(w)
    if w.dtype == np.float32:
        return w
    if w.dtype == np.uint16:
        return (w.astype(np.uint32) << 16).view(np.float32)
    raise TypeError("weights must be float32 or bfloat16 bits (uint16)")


def exact_abs_sum(w: np.ndarray) -> tuple[int, int]:
    """sum |w| exactly, as (num, e) with sum = num * 2**e (num a Python int).

    Every finite float32 is mant * 2**exp with an integer mant < 2**24;
    the terms are summed per exponent (int64 cannot overflow below 2**39
    terms) and the per-exponent sums are combined in Python integers."""
    a = np.abs(as_f32(w).astype(np.float64)).ravel()
    a = a[a != 0]
    if a.size == 0:
        return 0, 0
    frac, ex = np.frexp(a)                      # a = frac * 2**ex, 0.5 <= frac < 1
    mant = np.ldexp(frac, 24).astype(np.int64)  # exact: float32 has 24 bits
    ex = ex.astype(np.int64) - 24
    e0 = int(ex.min())
    total = 0
    for e in np.unique(ex):
        total += int(mant[ex == e].sum()) << (int(e) - e0)
    return total, e0


def round_ratio_f32(num: int, den: int) -> np.float32:
    """The float32 nearest to num / den (num >= 0, den > 0 integers), ties
    to even; values past the float32 range are not expected here."""
    if num == 0:
        return np.float32(0.0)
    # exponent q of the last kept bit: 24 significant bits for normal
    # results, the fixed quantum 2**-149 for subnormal ones
    lead = num.bit_length() - den.bit_length()  # floor(log2(num/den)) is lead or lead-1
    if (num << max(0, -lead)) < (den << max(0, lead)):
        lead -= 1
    q = max(lead - 23, -149)
    # m = num / den / 2**q, split into integer part and remainder
    n_, d_ = (num, den << q) if q >= 0 else (num << -q, den)
    m, r = divmod(n_, d_)
    if 2 * r > d_ or (2 * r == d_ and (m & 1)):
        m += 1
    return np.float32(np.ldexp(np.float64(m), q))


def abs_mean(w: np.ndarray) -> np.float32:
    """gamma = mean |W| (reading Q1)."""
    n = int(np.asarray(w).size)
    num, e = exact_abs_sum(w)
    if e >= 0:
        return round_ratio_f32(num << e, n)
    return round_ratio_f32(num, n << -e)


def abs_max(w: np.ndarray) -> np.float32:
    """max |W| ([I2S] "Per-Tensor Scaling Strategy")."""
    return np.float32(np.abs(as_f32(w)).max())


def round_clip(q: np.ndarray) -> np.ndarray:
    """RoundClip(q, -1, 1) = max(-1, min(1, round(q))), round half to even;
    NaN (0/0) -> 0 (reading Q3)."""
    q = np.where(np.isnan(q), np.float32(0), q)
    return np.clip(np.round(q), -1, 1).astype(np.int8)


def ternarize(w: np.ndarray, mode: str = ABSMEAN, eps: float = 0.0):
    """W [M, K] float32 (or bf16 bits) -> (codes int8 [M, K] in {-1, 0, 1},
    s, d): s the statistic (mean or max of |W|), d = float32(s + eps) the
    divisor and scale."""
    if not (np.isfinite(eps) and eps >= 0):
        raise ValueError("eps must be finite and >= 0")
    if mode not in (ABSMEAN, ABSMAX):
        raise ValueError(mode)
    w32 = as_f32(w)
    s = abs_mean(w32) if mode == ABSMEAN else abs_max(w32)
    d = np.float32(s + np.float32(eps))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = w32 / d                                 # float32 division
    return round_clip(q), s, d


def quantize_weights(w: np.ndarray, mode: str = ABSMEAN, eps: float = 0.0):
    """Ternarize and pack: (packed bytes with scale d in the tail, s, d)."""
    from . import pack
    codes, s, d = ternarize(w, mode, eps)
    packed, bad = pack(codes, float(d))
    assert bad == 0
    return packed, s, d
