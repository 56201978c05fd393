"""Exact rational statements of the bf16 format and of round-to-nearest-even,
written from the format's definition (1 sign bit, 8 exponent bits with bias
127, 7 fraction bits; subnormals below 2^-126).  Used by the oracle pins as a
check that shares nothing with the oracle's own C rounding."""
import math
from fractions import Fraction


def bf16_exact(b):
    """Exact value of a finite bf16 pattern as a Fraction, from the format."""
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(f, 128) * Fraction(2) ** -126
    return sign * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)


def rne_bf16_exact(v: Fraction, negative_zero=False):
    """Round an exact rational to bf16 (nearest, ties to even) -> pattern."""
    if v == 0:
        return 0x8000 if negative_zero else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # exponent of the leading bit
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)                    # quantum exponent
    n = a / Fraction(2) ** q
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * Fraction(2) ** q
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    if r < Fraction(2) ** -126:
        return sign | int(r / Fraction(2) ** -133)
    e2 = e if r < Fraction(2) ** (e + 1) else e + 1
    frac = int((r / Fraction(2) ** e2 - 1) * 128)
    return sign | ((e2 + 127) << 7) | frac
