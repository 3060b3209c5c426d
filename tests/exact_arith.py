"""Exact rational arithmetic for brute-force pins of the oracle.

Independent of the oracle's C converters: values are ``fractions.Fraction`` and rounding is
written here from the IEEE 754 definition (nearest representable value, ties to an even
significand, gradual underflow, overflow to infinity).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

# (stored significand bits, minimum normal exponent, maximum finite exponent)
FORMATS = {
    "fp32": (23, -126, 127),
    "fp16": (10, -14, 15),
    "bf16": (7, -126, 127),
}


def floor_log2(a: Fraction) -> int:
    """Largest e with 2**e <= a, for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_nearest_even(q: Fraction, fmt: str):
    """Round an exact rational to the format; returns a Fraction or +-math.inf."""
    p, emin, emax = FORMATS[fmt]
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(floor_log2(a), emin)          # below emin the quantum is fixed (subnormals)
    quantum = Fraction(2) ** (e - p)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    max_finite = (2 - Fraction(2) ** (-p)) * Fraction(2) ** emax
    if r > max_finite:
        return sign * math.inf
    return sign * r


def f32_value(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0])


def to_bits(value, fmt: str) -> int:
    """Encode an exactly representable value (Fraction or +-inf) in the format's bit pattern."""
    p, emin, emax = FORMATS[fmt]
    ebits = {"fp32": 8, "fp16": 5, "bf16": 8}[fmt]
    width = 1 + ebits + p
    if value == math.inf or value == -math.inf:
        return ((1 if value < 0 else 0) << (width - 1)) | (((1 << ebits) - 1) << p)
    value = Fraction(value)
    sign = 1 if value < 0 else 0
    a = abs(value)
    if a == 0:
        return sign << (width - 1)
    bias = (1 << (ebits - 1)) - 1
    e = floor_log2(a)
    if e < emin:
        n = a / Fraction(2) ** (emin - p)
        assert n.denominator == 1, "not representable"
        return (sign << (width - 1)) | int(n)
    n = a / Fraction(2) ** (e - p)
    assert n.denominator == 1 and n < 2 ** (p + 1), "not representable"
    return (sign << (width - 1)) | ((e + bias) << p) | (int(n) - (1 << p))


def from_bits(bits: int, fmt: str) -> Fraction:
    """Decode a finite bit pattern exactly."""
    p, emin, emax = FORMATS[fmt]
    ebits = {"fp32": 8, "fp16": 5, "bf16": 8}[fmt]
    width = 1 + ebits + p
    sign = -1 if (bits >> (width - 1)) & 1 else 1
    field = (bits >> p) & ((1 << ebits) - 1)
    frac = bits & ((1 << p) - 1)
    assert field != (1 << ebits) - 1, "inf/nan"
    if field == 0:
        return sign * Fraction(frac) * Fraction(2) ** (emin - p)
    bias = (1 << (ebits - 1)) - 1
    return sign * Fraction((1 << p) + frac) * Fraction(2) ** (field - bias - p)
