"""Exact-rational helpers for pinning the oracle (CPU only).

Everything here works on Python Fractions, so no floating-point rounding
enters an expected value except where a pin says so (fp32 underflow of a
quotient is decided by an exact comparison with 2^-150).
"""

from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str = "format_constants.json") -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        data = json.load(f)
    return {k: v["value"] for k, v in data.items() if not k.startswith("_")}


def bf16_fraction(h: int) -> Fraction | None:
    """Exact value of a bf16 bit pattern; None for NaN/Inf."""
    sign = -1 if h & 0x8000 else 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    if e == 0xFF:
        return None
    if e == 0:
        v = Fraction(m, 128) * Fraction(2) ** -126
    else:
        v = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return sign * v


def is_negative_bits(h: int) -> bool:
    return bool(h & 0x8000)


def ceil_log2(v: Fraction) -> int:
    """Smallest integer e with 2^e >= v > 0."""
    assert v > 0
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e < v:
        e += 1
    while Fraction(2) ** (e - 1) >= v:
        e -= 1
    return e


def midpoint_index(a: Fraction, mids, strict) -> int:
    """E2M1 magnitude index by counting passed midpoints, the comparison
    strictness alternating as the store page's `_quantize_e2m1` prints it."""
    idx = 0
    for m, s in zip(mids, strict):
        m = Fraction(m)
        idx += (a > m) if s else (a >= m)
    return idx


def fp32_quotient_is_zero(x: Fraction, e: int) -> bool:
    """Does RN_fp32(x / 2^e) underflow to (signed) zero?  True exactly when
    |x / 2^e| <= 2^-150 (half of the least subnormal; the tie goes to even,
    which is zero)."""
    return abs(x) / Fraction(2) ** e <= Fraction(2) ** -150


def bf16_bits_of_fraction(v: Fraction) -> int:
    """bf16 bits of an exactly representable value, or +-Inf at >= 2^128."""
    if abs(v) >= Fraction(2) ** 128:
        return 0xFF80 if v < 0 else 0x7F80
    f = float(v)
    assert Fraction(f) == v
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert u & 0xFFFF == 0, "not a bf16 value"
    return u >> 16


def f32(x) -> np.float32:
    return np.float32(x)


def f32_bits(x: np.float32) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])
