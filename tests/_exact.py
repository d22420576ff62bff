"""Exact rational helpers used by the oracle pins (brute force on tiny inputs).

They work on Python ``fractions.Fraction`` values and re-derive every quantity
from the raw bytes and bit patterns with loops, independently of the oracle's
vectorised numpy code.
"""
from __future__ import annotations

import struct
from fractions import Fraction as F


def f16_value(bits16: int) -> F:
    """Exact value of an IEEE binary16 bit pattern (finite only)."""
    bits16 &= 0xFFFF
    sign = -1 if bits16 >> 15 else 1
    e = (bits16 >> 10) & 0x1F
    m = bits16 & 0x3FF
    if e == 0x1F:
        raise ValueError("non-finite fp16")
    if e == 0:
        return sign * F(m, 1 << 24)
    return sign * F(1024 + m, 1024) * F(2) ** (e - 15)


def f32_value(x: float) -> F:
    """Exact value of a float32 given as a Python float that is float32-representable."""
    return F(struct.unpack("<f", struct.pack("<f", x))[0])


def bf16_value(bits16: int) -> F:
    u = (bits16 & 0xFFFF) << 16
    return F(struct.unpack("<f", struct.pack("<I", u))[0])


def rn32(x: F) -> F:
    """Round a rational to the nearest fp32 value, ties to even (normal and subnormal)."""
    if x == 0:
        return F(0)
    s = -1 if x < 0 else 1
    x = abs(x)
    e = 0
    while x >= 2:
        x /= 2
        e += 1
    while x < 1:
        x *= 2
        e -= 1
    shift = 23 if e >= -126 else 23 - (-126 - e)
    m = x * F(2) ** shift
    fl = m.numerator // m.denominator
    r = m - fl
    if r > F(1, 2) or (r == F(1, 2) and fl % 2):
        fl += 1
    return s * F(fl) * F(2) ** (e - shift)


def read_field(stream: bytes, bit_offset: int, width: int) -> int:
    """Unsigned value of `width` bits starting at bit_offset, LSB-first."""
    v = 0
    for i in range(width):
        p = bit_offset + i
        v |= ((stream[p // 8] >> (p % 8)) & 1) << i
    return v


def signed_code(field: int, width: int) -> int:
    return field - (1 << width) if field >> (width - 1) else field


def cubic_q(a: F, b: F, t: F) -> F:
    """q(t) = a t + b t^2 + (1 - a - b) t^3, evaluated directly."""
    return a * t + b * t * t + (1 - a - b) * t * t * t


def weight_value(k: int, s: F, a: F, b: F, bits: int) -> F:
    km = (1 << (bits - 1)) - 1
    if k == 0:
        return F(0)
    t = F(abs(k), km)
    mag = s * cubic_q(a, b, t)
    return mag if k > 0 else -mag


def rne_int(x: F) -> int:
    fl = x.numerator // x.denominator
    r = x - fl
    if r > F(1, 2) or (r == F(1, 2) and fl % 2):
        fl += 1
    return fl


def rn32_float32(x: F):
    """rn32 as a numpy float32: an exact zero is +0.0, a nonzero value that rounds
    to zero keeps its sign, a rounded magnitude of 2^128 or more is an infinity."""
    import numpy as np
    if x == 0:
        return np.float32(0.0)
    r = rn32(x)
    if abs(r) >= F(2) ** 128:
        return np.float32(np.inf) if x > 0 else np.float32(-np.inf)
    if r == 0:
        return np.float32(-0.0) if x < 0 else np.float32(0.0)
    return np.float32(float(r))


def nearest_code(w: F, s: F, a: F, b: F, bits: int) -> int:
    """Code k in [-Kmax, Kmax] whose fp32 level rn32(s sign(k) q(|k|/Kmax)) is
    nearest to w by exact distance; among equal distances the smaller |k|, then
    the first of k = +j, -j (equal distances at +j and -j need w = 0 or a zero
    level, and then k = 0 is at least as near)."""
    km = (1 << (bits - 1)) - 1
    best, best_k = None, 0
    for j in range(km + 1):
        for k in ((j, -j) if j else (0,)):
            lv = rn32(weight_value(k, s, a, b, bits))
            d = abs(w - lv)
            if best is None or d < best:
                best, best_k = d, k
    return best_k
