"""Exact rational arithmetic helpers for pinning the oracle (tests only).

Independent of the oracle's C code: values are decoded from their bit patterns
with integer arithmetic and rounded with integer arithmetic, so a mistake in
the oracle's own conversions cannot hide behind these helpers.
"""
from __future__ import annotations

from fractions import Fraction


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern (1 sign, 8 exponent, 7 fraction bits)."""
    bits &= 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    assert e != 0xFF, "non-finite"
    if e == 0:
        return sign * Fraction(f, 2 ** 133)
    return sign * Fraction(128 + f, 128) * Fraction(2) ** (e - 127)


def round_binary(v: Fraction, p: int, emin: int, emax: int):
    """Round v to the nearest binary float with p significand bits (ties to even).

    emin: exponent of the smallest normal; emax: exponent of the largest finite.
    Returns a Fraction, or +-inf as a float when it overflows.
    """
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (p - 1))
    units = a / ulp
    fl = units.numerator // units.denominator
    rem = units - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * r


def to_f32(v: Fraction):
    return round_binary(v, 24, -126, 127)


def to_bf16(v: Fraction):
    return round_binary(v, 8, -126, 127)


def bf16_bits_of(v: Fraction) -> int:
    """bf16 bit pattern of a value that is exactly representable in bf16."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    for e in range(1, 255):
        lo = Fraction(2) ** (e - 127)
        if lo <= a < 2 * lo:
            f = (a / lo - 1) * 128
            assert f.denominator == 1, "not representable"
            return sign | (e << 7) | int(f)
    f = a * 2 ** 133
    assert f.denominator == 1 and f < 128, "not representable"
    return sign | int(f)
