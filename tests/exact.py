"""Exact-arithmetic helpers for the CPU pins: fp32 rounding of a rational number and an
fp32 fused multiply-add written from their definitions (round-to-nearest, ties to even)."""
from fractions import Fraction

import numpy as np


def f32_round(x: Fraction) -> float:
    """Nearest fp32 to the exact rational x, ties to even (normal and subnormal range)."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q_exp = max(e - 23, -149)          # quantum of fp32 in this binade (subnormals: 2^-149)
    scaled = a / (Fraction(2) ** q_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(n * Fraction(2) ** q_exp)   # exact: n has at most 24 bits
    return float(np.float32(sign * v))


def fmaf(a: float, b: float, c: float) -> float:
    return f32_round(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def addf(a: float, b: float) -> float:
    return f32_round(Fraction(float(a)) + Fraction(float(b)))
