"""Q8 of one block in exact rational arithmetic, for deriving and re-checking
the hand-worked golden lines of q8_tiny.txt.

Every fp32 step of the Q8 definition (d = amax / 127, r = 1 / d, id = r when r
is finite else 0, t = v * id, q = rint(t) clamped to +-127) is carried out on
Fractions and rounded to the nearest fp32 value (ties to even, subnormals kept,
overflow to infinity) explicitly, so the result does not depend on any float
unit, compiler or library.  It imports nothing from the oracle or the library.
"""
from __future__ import annotations

import struct
from fractions import Fraction

INF = float("inf")


def f32_bits(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def from_bits(b: int) -> Fraction:
    """The exact value of an fp32 bit pattern (finite patterns only)."""
    sign = -1 if b >> 31 else 1
    e = (b >> 23) & 0xFF
    m = b & 0x7FFFFF
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(m, 1 << 149)
    return sign * Fraction((1 << 23) | m) * Fraction(2) ** (e - 150)


def round_f32(x: Fraction):
    """Nearest fp32 value of x (ties to even), as a Fraction, or +-inf."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)   # subnormal spacing below 2^-126
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    v = k * quantum
    if v >= Fraction(2) ** 128:
        return sign * INF
    return sign * v


def rint_even(t: Fraction) -> int:
    k = t.numerator // t.denominator
    rem = t - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return k


def q8_exact(values):
    """(q list, d as a Fraction, qsum) of one block of exact fp32 values."""
    amax = max(abs(v) for v in values)
    d = round_f32(amax / 127)
    r = round_f32(1 / d) if d != 0 else INF
    inv = Fraction(0) if r in (INF, -INF) else r
    q = [max(-127, min(127, rint_even(round_f32(v * inv)))) for v in values]
    return q, d, sum(q)
