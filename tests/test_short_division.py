"""The scale fit's reciprocals and quotients (csrc/stq_device.h: recip_h,
div_h, div_qmax), replayed in exact rational arithmetic on the host.

The kernels replace IEEE divisions whose operands have at most 11 significant
bits (fp16 values, 7, 31, 127) by a reciprocal estimate, one Newton step and
one quotient correction.  The claim is that the result is the correctly
rounded quotient for every such operand, whenever the estimate is within one
ulp of 1/b.  These tests replay the steps with exact fractions (each fma
rounded once to fp32), with the estimate taken one ulp low, exact and one ulp
high, and compare with the correctly rounded quotient: every positive finite
fp16 divisor for the reciprocal, and seeded samples for the quotients.
"""
from fractions import Fraction

import numpy as np
import pytest


def rn32(x: Fraction) -> Fraction:
    """x rounded to the nearest fp32 value, ties to even (no overflow here)."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                     # subnormals share the exponent of 2^-126
    q = a / Fraction(2) ** (e - 23)      # significand scaled to an integer part of 24 bits
    n, r = divmod(q.numerator, q.denominator)
    rem = Fraction(r, q.denominator)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * Fraction(n) * Fraction(2) ** (e - 23)


def ulp32(x: Fraction) -> Fraction:
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    return Fraction(2) ** (max(e, -126) - 23)


def fma32(a, b, c):
    return rn32(a * b + c)


def recip_h(b: Fraction, r: Fraction) -> Fraction:
    e = fma32(-b, r, Fraction(1))
    return fma32(e, r, r)


def div_h(a: Fraction, b: Fraction, r: Fraction) -> Fraction:
    y = recip_h(b, r)
    q = rn32(a * y)
    return fma32(fma32(-b, q, a), y, q)


def estimates(b: Fraction):
    """Reciprocal estimates within one ulp of 1/b."""
    t = rn32(1 / b)
    return (t - ulp32(t), t, t + ulp32(t))


def fp16_values():
    bits = np.arange(1, 0x7C00, dtype=np.uint16)  # every positive finite fp16
    return [Fraction(float(v)) for v in bits.view(np.float16).astype(np.float64)]


def test_reciprocal_of_every_fp16_value():
    for b in fp16_values():
        want = rn32(1 / b)
        for r in estimates(b):
            assert recip_h(b, r) == want, (b, r)


def test_quotients_of_fp16_values():
    vals = fp16_values()
    rng = np.random.default_rng(5)
    pairs = rng.integers(0, len(vals), (6000, 2))
    extra = [(0, 0), (len(vals) - 1, 0), (0, len(vals) - 1)]
    for i, j in list(map(tuple, pairs)) + extra:
        a, b = vals[i], vals[j]
        want = rn32(a / b)
        for r in estimates(b):
            assert div_h(a, b, r) == want, (a, b, r)
    # 1 / c (pack and the window end) and s / c with s = 1
    for b in vals[::7]:
        assert div_h(Fraction(1), b, rn32(1 / b)) == rn32(1 / b)


@pytest.mark.parametrize("w,n", [(4, 7), (6, 31), (8, 127)])
def test_row_step_quotient(w, n):
    """RN(a / n) for fp32 a of every magnitude class: normal, subnormal, near
    the top of the range, and values a/n that are floats themselves."""
    rng = np.random.default_rng(w)
    raw = rng.integers(1, 0x7F7FFFFF, 4000, dtype=np.uint32)
    raw = np.concatenate([raw, rng.integers(1, 0x00800000, 300, dtype=np.uint32)])
    xs = [Fraction(float(v)) for v in raw.view(np.float32).astype(np.float64)]
    xs += [Fraction(n * k) for k in (1, 3, 1024, 12345)]
    y = rn32(Fraction(1, n))
    for a in xs:
        q = rn32(a * y)
        got = fma32(fma32(Fraction(-n), q, a), y, q)
        assert got == rn32(a / n), (a, n)
