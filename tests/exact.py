"""Exact rational arithmetic for pinning the oracle (tests only).

Everything here works on Python ``Fraction``s and integers, so it shares no
floating-point code path with NumPy; a float32 result is produced by an
explicit round-to-nearest-even of the exact rational.
"""
from fractions import Fraction

import numpy as np


def F(x) -> Fraction:
    """Exact rational value of a float / numpy float / int."""
    return Fraction(float(x)) if not isinstance(x, (int, Fraction)) else Fraction(x)


def rint_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (RN-even) binary32 value of an exact rational, subnormals included."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = _floor_log2(a)
    qexp = max(e, -126) - 23          # spacing of binary32 numbers around a
    quantum = Fraction(2) ** qexp
    n = rint_half_even(a / quantum)
    val = n * quantum
    if val >= Fraction(2) ** 128:
        raise OverflowError("rounds past the float32 range")
    return np.float32(sign * float(val))


def f32_bits(x) -> int:
    return int(np.float32(x).view(np.uint32))


def fma_f32(a, b, c) -> np.float32:
    return round_f32(F(a) * F(b) + F(c))


def quant_rule_exact(row):
    """Per-row absmax INT8 rule evaluated with exact rationals + explicit rounding.

    Returns (q list[int], scale np.float32)."""
    amax = max((abs(F(v)) for v in row), default=Fraction(0))
    if amax == 0:
        return [0] * len(row), np.float32(0.0)
    s = round_f32(amax / 127)
    q = []
    for v in row:
        t = round_f32(F(v) / F(s))
        q.append(max(-127, min(127, rint_half_even(F(t)))))
    return q, s
