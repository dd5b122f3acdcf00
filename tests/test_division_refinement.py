"""The division-free group quantisation of the GPU kernels, replayed in exact arithmetic.

The kernels quantise a group against its scale s = RN(amax/127) with
y = RN(1/s) and two fused residual corrections instead of one IEEE division
per element, then round to an integer by adding 1.5*2^23. This test replays
that sequence with exact rationals and an explicit binary32 round-to-nearest
after every operation (a fused multiply-add rounds once), and checks the
result against RN(x/s) and against the absmax rule's code. Besides random
groups it places quotients next to half-integers, where a quotient that is
only faithful (not correctly rounded) would change the integer code, and it
covers decoded block-format values, whose quotients land at exactly such
points (x = amax/2 gives x/s = 63.5 up to the rounding of s).
"""
from fractions import Fraction

import numpy as np
import pytest

from tests.exact import F, round_f32, rint_half_even

FAST_MIN = Fraction(1, 2 ** 100)
ROUND = Fraction(12582912)                 # 1.5 * 2^23


def rn(v: Fraction) -> Fraction:
    return F(round_f32(v))


def refined_code(x: Fraction, s: Fraction, y: Fraction) -> int:
    q = rn(x * y)
    q = rn(q + y * rn(x - s * q))           # fma(fma(-s, q, x), y, q)
    q2 = rn(q + y * rn(x - s * q))
    t = rn(q2 + ROUND)                      # the integer lands in the low bits
    return int(t - ROUND), q2


def rule_code(x: Fraction, s: Fraction) -> int:
    return max(-127, min(127, rint_half_even(rn(x / s))))


def check_group(vals):
    vals = [F(np.float32(v)) for v in vals]
    amax = max(abs(v) for v in vals)
    s = rn(amax / 127)
    assert s >= FAST_MIN
    y = rn(1 / s)
    for x in vals:
        code, q2 = refined_code(x, s, y)
        assert q2 == rn(x / s), (float(x), float(s))
        assert code == rule_code(x, s), (float(x), float(s))
        assert -127 <= code <= 127


def test_random_groups():
    rng = np.random.default_rng(7)
    for _ in range(40):
        e = int(rng.integers(-90, 90))
        g = (rng.standard_normal(32) * 2.0 ** e).astype(np.float32)
        check_group(g)


def test_quotients_next_to_half_integers():
    rng = np.random.default_rng(8)
    for _ in range(60):
        amax = np.float32(abs(rng.standard_normal()) * 2.0 ** int(rng.integers(-60, 60)) + 1e-30)
        s = rn(F(amax) / 127)
        vals = [amax]
        for _ in range(6):
            k = int(rng.integers(-127, 127))
            target = np.float32(float(s * (Fraction(2 * k + 1, 2))))
            for d in (-2, -1, 0, 1, 2):     # the float neighbours of s*(k + 1/2)
                v = np.nextafter(target, np.float32(np.inf) if d > 0 else np.float32(-np.inf))
                for _ in range(abs(d) - 1 if d else 0):
                    v = np.nextafter(v, np.float32(np.inf) if d > 0 else np.float32(-np.inf))
                v = target if d == 0 else v
                if abs(v) <= amax:
                    vals.append(v)
        check_group(vals)


@pytest.mark.parametrize("ocp_max", [448.0, 240.0])
def test_decoded_block_values(ocp_max):
    """Every e4m3 magnitude times a few power-of-two block scales, against the
    group maxima that decoded weights produce (the quotients 127*m/M)."""
    mags = sorted({float(m * 2.0 ** e) for m in range(8, 16) for e in range(-9, 9)
                   if m * 2.0 ** e <= ocp_max} | {float(m) * 2.0 ** -9 for m in range(1, 8)})
    for amax in (mags[-1], 416.0, 240.0, 1.0, 0.75, 2.0 ** -9 * 7):
        for scale_e in (-20, 0, 37):
            vals = [m * 2.0 ** scale_e for m in mags if m <= amax]
            vals = vals + [-v for v in vals]
            check_group(vals)
