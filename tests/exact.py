"""Exact rational arithmetic helpers for the oracle's pins (no floating-point
library routine involved): correctly rounded binary32 of a rational, and
round-half-to-even to an integer."""
from fractions import Fraction


def round_to_f32(fr: Fraction) -> float:
    """The binary32 value nearest to the exact rational ``fr`` (ties to even).
    Normal and subnormal ranges; raises on overflow."""
    fr = Fraction(fr)
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** E > a:
        E -= 1
    while Fraction(2) ** (E + 1) <= a:
        E += 1
    E = max(E, -126)                       # below 2^-126 the spacing stays 2^-149
    quantum = Fraction(2) ** (E - 23)
    t = a / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** 128:
        raise OverflowError
    return sign * float(val)               # val is a binary32 value, so float() is exact


def round_to_f16(fr: Fraction) -> float:
    """The binary16 value nearest to ``fr`` (ties to even); inf on overflow."""
    fr = Fraction(fr)
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** E > a:
        E -= 1
    while Fraction(2) ** (E + 1) <= a:
        E += 1
    E = max(E, -14)
    quantum = Fraction(2) ** (E - 10)
    t = a / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val > 65504:
        return sign * float("inf")
    return sign * float(val)


def rne_int(fr) -> int:
    """Nearest integer to an exact rational (or a float, taken exactly), ties to even."""
    fr = Fraction(fr)
    n = fr.numerator // fr.denominator
    rem = fr - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n
