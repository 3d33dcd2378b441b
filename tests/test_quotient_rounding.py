"""The epilogues' x / b (struct Quotient in csrc/common.h), emulated exactly on the CPU.

The device code computes one reciprocal r of b (v_rcp_f32, within one ulp of 1/b), refines it
with one Newton step y = fma(fma(-b, r, 1), r, r), and then, for every x, q = x*y and
q' = fma(fma(-b, q, x), y, q): Markstein's final division step.  Every step rounds to fp32
once (RNE); here each is computed exactly with rationals and rounded to fp32 by hand, for r
equal to the correctly rounded 1/b and to both of its neighbours, and q' is compared with
the correctly rounded x / b, which the division it replaces returns.  The ranges are the
epilogues': b is a row sum within a few binades of 1, x an accumulated output.
"""
import math
import random
from fractions import Fraction

import pytest


def rn32(v):
    """Round a rational to the nearest fp32 value, ties to even (normal range)."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2^23 <= a / 2^(e-23) < 2^24
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    scale = Fraction(2) ** (e - 23)
    m = a / scale
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * scale


def ulp32(v):
    a = abs(Fraction(v))
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    return Fraction(2) ** (e - 23)


def fma32(a, b, c):
    return rn32(Fraction(a) * Fraction(b) + Fraction(c))


def quotient(x, b, r):
    y = fma32(fma32(-b, r, 1), r, r)
    q = rn32(Fraction(x) * y)
    return fma32(fma32(-b, q, x), y, q)


def test_markstein_step_rounds_like_the_division():
    rng = random.Random(20261203)
    bad = []
    for _ in range(3000):
        b = rn32(Fraction(2) ** rng.uniform(-2, 24))
        x = rn32((1 if rng.random() < 0.5 else -1) * b * Fraction(2) ** rng.uniform(-12, 10))
        want = rn32(Fraction(x) / b)
        r0 = rn32(1 / Fraction(b))
        for r in (r0, r0 + ulp32(r0), r0 - ulp32(r0)):
            got = quotient(x, b, r)
            if got != want:
                bad.append((float(x), float(b), float(r), float(got), float(want)))
    assert not bad, bad[:5]


def test_exact_quotients_stay_exact():
    # row 0 sees one key: O = p * v and L = p, so O / L must return v exactly
    rng = random.Random(7)
    for _ in range(2000):
        p = rn32(Fraction(rng.randint(8, 15), 8) * Fraction(2) ** rng.randint(4, 7))   # e4m3 values 128..240
        v = rn32(Fraction(rng.randint(-15, 15), 8) * Fraction(2) ** rng.randint(-6, 8))
        if v == 0:
            continue
        r0 = rn32(1 / Fraction(p))
        for r in (r0, r0 + ulp32(r0), r0 - ulp32(r0)):
            assert quotient(rn32(p * v), p, r) == v


@pytest.mark.parametrize("x", [0.0, 3.5, -2.0])
def test_row_without_keys_gives_zero(x):
    # b = infinity: the device code uses y = 0 and b = 0 in the residual, so q' = x * 0 + 0 = 0
    y, b = Fraction(0), Fraction(0)
    q = rn32(Fraction(x) * y) if x else Fraction(0)
    assert fma32(fma32(-b, q, 0), y, q) == 0
