"""Pins of the GEMM acceptance rule in tests/parity.py (CPU only).

The rule holds a GPU result g against the oracle's exact value y with the bound
b = 2^-8 |y| + 1e-6 sum|a w|, and extends it to the ends of BF16's range: the
correctly rounded BF16 result of y must always be accepted, including +-inf when y
lies beyond BF16's finite range and +-0 (or a subnormal) when y lies in or below the
subnormal range.  The expected verdicts here are worked out by hand from the BF16
format (8 exponent bits, 7 stored significand bits, largest finite (2 - 2^-7) 2^127,
smallest subnormal 2^-133); the last test checks every verdict against torch's own
float64 -> bfloat16 rounding, a library routine independent of the rule's formula.
"""
import numpy as np
import pytest

from parity import BF16_MAX, BF16_OVERFLOW, gemm_accepts, gemm_within_tolerance

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
INF = float("inf")


def verdict(g, y, ad):
    ok, _ = gemm_accepts(np.array([g]), np.array([y]), np.array([ad]))
    return bool(ok[0])


def test_constants_of_the_bf16_format():
    assert BF16_MAX == 3.3895313892515355e38                  # 0x7F7F
    assert BF16_OVERFLOW == 2.0 ** 128 - 2.0 ** 119           # halfway between 0x7F7F and 2^128


def test_normal_range_is_the_literal_bound():
    assert verdict(1.0, 1.0, 1.0)
    assert verdict(1.0 + 2.0 ** -8, 1.0, 0.0)                 # err == 2^-8 |y|: on the bound
    assert not verdict(1.0 + 2.0 ** -7, 1.0, 0.0)             # next BF16 up: twice the bound
    assert verdict(1.0 + 2.0 ** -7, 1.0, 2.0 ** -7 / 1e-6)    # absolute term covers it
    assert not verdict(-1.0, 1.0, 1.0)                        # sign error
    assert not verdict(1.0, 0.0, 1.0)                         # cancellation: bound is 1e-6


def test_overflow_to_infinity():
    y = 2.0 ** 130                                            # beyond BF16's range: the answer is +inf
    assert verdict(INF, y, y)
    assert not verdict(BF16_MAX, y, y)                        # 3 * 2^128 away
    assert not verdict(-INF, y, y)
    assert verdict(-INF, -y, y)
    assert not verdict(INF, -y, y)
    # exactly representable value below the threshold, band does not reach it: inf is wrong
    y = 2.0 ** 128 - 2.0 ** 121
    assert verdict(y, y, y)
    assert not verdict(INF, y, y)
    # the threshold itself is a tie that rounds to inf; the largest finite value is within the band too
    assert verdict(INF, BF16_OVERFLOW, 0.0)
    assert verdict(BF16_MAX, BF16_OVERFLOW, 0.0)
    # a value just below the threshold whose band crosses it: both answers accepted
    y = BF16_OVERFLOW * (1 - 2.0 ** -12)
    assert verdict(INF, y, 0.0) and verdict(BF16_MAX, y, 0.0)


def test_underflow_to_zero_and_gradual_underflow():
    assert verdict(0.0, 2.0 ** -140, 2.0 ** -140)             # below half the smallest subnormal: 0
    assert verdict(-0.0, 2.0 ** -140, 2.0 ** -140)
    assert verdict(0.0, -2.0 ** -135, 0.0)
    assert not verdict(2.0 ** -132, 2.0 ** -140, 2.0 ** -140)  # two subnormal steps away
    assert verdict(2.0 ** -130, 2.0 ** -130, 2.0 ** -130)     # a representable subnormal
    assert not verdict(0.0, 2.0 ** -130, 2.0 ** -130)         # flushing it to zero is wrong
    tie = 1.5 * 2.0 ** -133                                   # halfway between 2^-133 and 2^-132
    assert verdict(2.0 ** -132, tie, 0.0) and verdict(2.0 ** -133, tie, 0.0)
    assert not verdict(2.0 ** -131, tie, 0.0)
    assert not verdict(0.0, 2.0 ** -126, 2.0 ** -126)         # smallest normal: not zero


def test_nan_handling():
    nan = float("nan")
    assert verdict(nan, nan, nan)
    assert not verdict(0.0, nan, nan)
    assert not verdict(nan, 1.0, 1.0)
    assert not verdict(INF, nan, nan)


def test_ratio_and_counts():
    ok, ratio, nbad = gemm_within_tolerance(np.array([1.0, INF, 2.0]), np.array([1.0, 2.0 ** 131, 1.0]),
                                            np.array([0.0, 0.0, 0.0]))
    assert not ok and nbad == 1 and ratio == pytest.approx(1.0 / (2.0 ** -8 + 2.0 ** -134))


def test_correctly_rounded_result_is_always_accepted():
    """torch's float64 -> bfloat16 cast (round to nearest even, overflow to inf, gradual
    underflow) of exact values spread over the whole exponent range, including both
    ends, is accepted with no absolute term; one BF16 step beyond it in the normal range
    is not."""
    import torch
    rng = np.random.default_rng(5)
    e = rng.uniform(-150.0, 131.0, 20000)
    y = np.sign(rng.standard_normal(e.size)) * (1.0 + rng.random(e.size)) * 2.0 ** e
    y = np.concatenate([y, [BF16_OVERFLOW, -BF16_OVERFLOW, 2.0 ** -134, 1.5 * 2.0 ** -133, 0.0]])
    g = torch.from_numpy(y).to(torch.bfloat16).to(torch.float64).numpy()
    ok, _ = gemm_accepts(g, y, np.zeros_like(y))
    assert ok.all(), y[~ok][:5]
    normal = np.isfinite(g) & (np.abs(g) >= 2.0 ** -120) & (np.abs(g) <= 2.0 ** 126)
    up = torch.from_numpy(g[normal]).to(torch.bfloat16).view(torch.int16)
    # two BF16 steps away from the correctly rounded value (same sign, larger magnitude)
    far = (up + 2).view(torch.bfloat16).to(torch.float64).numpy()
    ok, _ = gemm_accepts(far, y[normal], np.zeros(normal.sum()))
    assert not ok.any()
