"""Exact-rational rounding helpers for the tests (independent of numpy's casts).

Round a Fraction to a binary floating-point format with p significand bits,
minimum normal exponent emin and round-to-nearest-even, from the definition of
such a format.  Used to pin the oracle's fp32 divisions and fp16 / E4M3
conversions against first principles.
"""
from fractions import Fraction
import math


def round_to_format(x: Fraction, p: int, emin: int, emax_val: Fraction = None) -> Fraction:
    """Nearest value of the format (ties to even significand). No overflow handling unless emax_val given (saturate)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                        # subnormals share the minimum exponent's spacing
    ulp = Fraction(2) ** (e - (p - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * ulp
    if emax_val is not None and v > emax_val:
        v = emax_val
    return sign * v


def rn_fp32(x: Fraction) -> Fraction:
    return round_to_format(x, 24, -126)


def rn_fp16(x: Fraction) -> Fraction:
    return round_to_format(x, 11, -14)


def rn_e4m3_sat(x: Fraction) -> Fraction:
    return round_to_format(x, 4, -6, Fraction(448))


def rint_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl
