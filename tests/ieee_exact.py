"""Exact IEEE-754 rounding on rational numbers, written from the standard's definition.

Used by the CPU tests to re-derive bit-exact float steps independently of NumPy's
float arithmetic: every value is a Fraction and every rounding is explicit.
"""

from fractions import Fraction
import math

INF = math.inf


def _exp2_floor(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_even_int(x: Fraction) -> int:
    f = math.floor(x)
    r = x - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def rne(x: Fraction, p: int, emin: int, emax: int):
    """Round x to the binary format with p significand bits and exponent range [emin, emax]."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_exp2_floor(a), emin)
    ulp = Fraction(2) ** (e - (p - 1))
    m = round_even_int(a / ulp)
    r = m * ulp
    maxf = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > maxf:
        return sign * INF
    return sign * r


def f32(x):
    return rne(Fraction(x), 24, -126, 127)


def f16(x):
    return rne(Fraction(x), 11, -14, 15)


def bf16(x):
    return rne(Fraction(x), 8, -126, 127)
