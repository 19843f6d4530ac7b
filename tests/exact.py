"""Exact rational arithmetic for pinning the oracle.

An independent formulation of round-to-nearest-even to BF16: decode the
value exactly as a Fraction, divide by the BF16 quantum of its binade
(2^(e-7), with e clamped to the smallest normal exponent -126 so subnormals
share the min-normal quantum), round the quotient with Python's
round-half-to-even on Fractions, and map values at or beyond 2^128 to
infinity.  Nothing here mirrors the oracle's nearest-of-two-candidates
code.
"""
from __future__ import annotations

import struct
from fractions import Fraction

NAN = "nan"


def f32_fraction(bits: int):
    """Exact value of an F32 bit pattern: Fraction, +-inf as float, or NAN."""
    sign = -1 if bits >> 31 else 1
    exp = (bits >> 23) & 0xFF
    man = bits & 0x7FFFFF
    if exp == 0xFF:
        return NAN if man else float("inf") * sign
    if exp == 0:
        return sign * Fraction(man, 1 << 149)
    return sign * Fraction(0x800000 | man) * Fraction(2) ** (exp - 150)


def bf16_fraction(bits: int):
    return f32_fraction((bits & 0xFFFF) << 16)


def _floor_log2(x: Fraction) -> int:
    """floor(log2(x)) for a positive Fraction."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    # 2^e <= x < 2^(e+1) after at most one correction either way
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def _encode_bf16_exact(v: Fraction, negative: bool) -> int:
    """BF16 bits of a value that is exactly representable (or 2^128 -> inf)."""
    if v == 0:
        return 0x8000 if negative else 0x0000
    if v >= Fraction(2) ** 128:
        return 0xFF80 if negative else 0x7F80
    f = float(v)  # exact: representable in binary32 hence in binary64
    assert Fraction(f) == v
    b32 = struct.unpack("<I", struct.pack("<f", f))[0]
    assert b32 & 0xFFFF == 0, hex(b32)
    return (b32 >> 16) | (0x8000 if negative else 0)


def rne_bf16_of_value(x) -> int:
    """BF16 bits nearest to an exact value x (ties to even), NaN -> 0x7FC0."""
    if x is NAN:
        return 0x7FC0
    if isinstance(x, float):  # infinity
        return 0x7F80 if x > 0 else 0xFF80
    negative = x < 0
    mag = -x if x < 0 else x
    if mag == 0:
        return 0x0000  # a signed zero is decided by the caller
    e = max(_floor_log2(mag), -126)
    quantum = Fraction(2) ** (e - 7)
    q = round(mag / quantum)  # Fraction.__round__ rounds half to even
    return _encode_bf16_exact(q * quantum, negative)


def rne_bf16_of_f32_bits(bits: int) -> int:
    x = f32_fraction(bits)
    if x is not NAN and not isinstance(x, float) and x == 0:
        return (bits >> 16) & 0x8000
    r = rne_bf16_of_value(x)
    # a nonzero value that rounds to zero keeps its sign
    if r == 0 and (bits >> 31):
        return 0x8000
    return r


def exact_sum_bf16(a: int, b: int):
    """Exact sum of two BF16 values, with IEEE rules for infinities/NaN and
    for the sign of an exact zero sum (round to nearest: +0 unless both
    operands are -0)."""
    x, y = bf16_fraction(a), bf16_fraction(b)
    if x is NAN or y is NAN:
        return NAN
    if isinstance(x, float) or isinstance(y, float):
        xs = x if isinstance(x, float) else 0.0
        ys = y if isinstance(y, float) else 0.0
        if isinstance(x, float) and isinstance(y, float) and xs != ys:
            return NAN
        return xs if isinstance(x, float) else ys
    return x + y


def f32_bits_of_exact_sum_rounded(a: int, b: int) -> int:
    """IEEE binary32 round-to-nearest-even of the exact BF16 sum, as bits,
    NaN canonical 0x7FC00000.  Independent of the oracle: quantize with
    round-half-even on Fractions in binary32's grid (24-bit significand,
    min normal exponent -126)."""
    s = exact_sum_bf16(a, b)
    if s is NAN:
        return 0x7FC00000
    if isinstance(s, float):
        return 0x7F800000 if s > 0 else 0xFF800000
    if s == 0:
        both_neg = (a & 0x8000) and (b & 0x8000)
        return 0x80000000 if both_neg else 0
    neg = s < 0
    mag = -s if neg else s
    e = max(_floor_log2(mag), -126)
    quantum = Fraction(2) ** (e - 23)
    v = round(mag / quantum) * quantum
    if v >= Fraction(2) ** 128:
        return 0xFF800000 if neg else 0x7F800000
    if v == 0:
        return 0x80000000 if neg else 0
    bits = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    return bits | (0x80000000 if neg else 0)


def bf16_bits_of_exact_sum(a: int, b: int) -> int:
    """BF16 RNE of the exact sum (one rounding)."""
    s = exact_sum_bf16(a, b)
    if s is NAN:
        return 0x7FC0
    if isinstance(s, float):
        return 0x7F80 if s > 0 else 0xFF80
    if s == 0:
        both_neg = (a & 0x8000) and (b & 0x8000)
        return 0x8000 if both_neg else 0
    r = rne_bf16_of_value(s)
    if r == 0 and s < 0:
        return 0x8000
    return r


def exact_sum_f32(a: int, b: int):
    """Exact sum of two F32 values given as bit patterns, with the IEEE rules
    for infinities and NaN (the sign of an exact zero is the caller's)."""
    x, y = f32_fraction(a), f32_fraction(b)
    if x is NAN or y is NAN:
        return NAN
    if isinstance(x, float) or isinstance(y, float):
        if isinstance(x, float) and isinstance(y, float) and x != y:
            return NAN
        return x if isinstance(x, float) else y
    return x + y


def f32_bits_of_exact_f32_sum(a: int, b: int) -> int:
    """IEEE binary32 round-to-nearest-even of the exact sum of two F32
    values, as bits; NaN canonical 0x7FC00000; an exact zero sum is +0 unless
    both operands are -0.  Quantised with round-half-even on Fractions in
    binary32's grid, as f32_bits_of_exact_sum_rounded does for BF16 inputs."""
    s = exact_sum_f32(a, b)
    if s is NAN:
        return 0x7FC00000
    if isinstance(s, float):
        return 0x7F800000 if s > 0 else 0xFF800000
    if s == 0:
        return 0x80000000 if (a >> 31) and (b >> 31) else 0
    neg = s < 0
    mag = -s if neg else s
    e = max(_floor_log2(mag), -126)
    quantum = Fraction(2) ** (e - 23)
    v = round(mag / quantum) * quantum
    if v >= Fraction(2) ** 128:
        return 0xFF800000 if neg else 0x7F800000
    if v == 0:
        return 0x80000000 if neg else 0
    bits = struct.unpack("<I", struct.pack("<f", float(v)))[0]
    return bits | (0x80000000 if neg else 0)
