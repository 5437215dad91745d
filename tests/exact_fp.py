"""Exact IEEE-754 rounding on rational numbers, for the oracle's operation-order pins.

Every value is a ``fractions.Fraction``; ``fl32`` / ``fl64`` round a rational to
the nearest binary32 / binary64 value with ties to even (the IEEE default mode),
and ``sqrt64`` is the correctly rounded binary64 square root. With these a pin
can derive, step by step and with no floating-point hardware involved, the
exact bits that a stated sequence of roundings must produce.

The module holds no part of the oracle and imports nothing from it.
"""
import math
import struct
from fractions import Fraction


def _round_bits(x, p, emin):
    """x rounded to a binary format with p significand bits and minimum normal
    exponent emin (subnormals included), ties to even. Overflow is not handled
    (no pin comes near it)."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # e = floor(log2(a))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - p + 1)
    n, rem = divmod(a, quantum)  # n integer part, rem in [0, quantum)
    n = int(n)
    half = quantum / 2
    if rem > half or (rem == half and n % 2 == 1):
        n += 1
    return sign * n * quantum


def fl32(x):
    return _round_bits(x, 24, -126)


def fl64(x):
    return _round_bits(x, 53, -1022)


def sqrt64(x):
    """Correctly rounded binary64 square root of a non-negative rational."""
    x = Fraction(x)
    if x < 0:
        raise ValueError("sqrt of a negative value")
    if x == 0:
        return Fraction(0)
    # r = floor(sqrt(x) * 2^s) = isqrt(floor(x * 4^s)), so sqrt(x) lies in
    # [lo, lo + 2^-s) with lo = r / 2^s. With sqrt(x) = 2^e * (1 + f), the
    # binary64 rounding midpoints are multiples of 2^(e - 53); s >= 53 - e puts
    # them on the 2^-s grid, so none lies strictly inside the interval and every
    # point of (lo, lo + 2^-s) rounds alike. e >= (num_bits - den_bits - 2) / 2,
    # which the choice of s below covers with a wide margin.
    s = 80 + max(0, x.denominator.bit_length() - x.numerator.bit_length())
    scaled = x * Fraction(4) ** s
    n = scaled.numerator // scaled.denominator
    r = math.isqrt(n)
    lo = Fraction(r, 2 ** s)
    if scaled.denominator == 1 and r * r == n:  # sqrt(x) == lo exactly
        return fl64(lo)
    return fl64(lo + Fraction(1, 2 ** (s + 1)))


def rne_int(x):
    """Round a rational to the nearest integer, ties to even."""
    x = Fraction(x)
    n = math.floor(x)
    rem = x - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return int(n)


def f32(v):
    """The exact rational value of a binary32 number given as a Python float."""
    return Fraction(struct.unpack("<f", struct.pack("<f", v))[0])


def bits32(q):
    """binary32 bit pattern of a rational that is exactly representable."""
    v = float(q)
    assert Fraction(v) == q, "not representable in binary64"
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    assert Fraction(struct.unpack("<f", struct.pack("<I", b))[0]) == q, "not representable in binary32"
    return b
