"""Exact-rational model of IEEE binary32 arithmetic, used only to pin the oracle's quantizer.

Each operation is evaluated exactly with fractions.Fraction and then rounded once to the
nearest binary32 value, ties to even -- the IEEE 754 definition of a correctly rounded
operation.  It shares nothing with numpy's float32 kernels, so agreement pins the oracle's
claim that every quantizer step is a single correctly rounded fp32 operation.
"""

from __future__ import annotations

import struct
from fractions import Fraction

_HALF = Fraction(1, 2)


def round_f32(x: Fraction) -> Fraction:
    """Nearest binary32 value to the rational x (ties to even).  Overflow is not modelled."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 23, -149)                     # spacing of binary32 values around a
    scaled = a / (Fraction(2) ** q)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > _HALF or (rem == _HALF and m % 2 == 1):
        m += 1
    return sign * m * Fraction(2) ** q


def rint_half_even(x: Fraction) -> int:
    m = x.numerator // x.denominator
    rem = x - m
    if rem > _HALF or (rem == _HALF and m % 2 == 1):
        m += 1
    return int(m)


def bf16_to_fraction(bits: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    return Fraction(f)


def f32_bits(x: Fraction) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def quantize_group_exact(bits_list, b: int):
    """Eq. (4) on one group, each step a correctly rounded binary32 operation (see oracle)."""
    xs = [bf16_to_fraction(v) for v in bits_list]
    if b == 16:
        return [int(v) for v in bits_list], Fraction(1), Fraction(0)
    mx, mn = max(xs), min(xs)
    z = mn                                      # +0 after canonicalisation
    n = Fraction(2 ** b - 1)
    R = round_f32(mx - mn)
    s = round_f32(R / n)
    if s == 0:
        return [0] * len(xs), s, z
    codes = []
    for x in xs:
        d = round_f32(x - z)
        r = round_f32(d / s)
        codes.append(rint_half_even(r))
    return codes, s, z
