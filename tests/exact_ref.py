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


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def check_bf16_rounding(got_bits: np.ndarray, exact: np.ndarray, band: float = 2.0 ** -10) -> int:
    """Check bf16 results against exact (float64) values computed in higher
    precision.  A result must be the round-to-nearest-even of the exact value,
    except where the exact value lies within ``band`` bf16 ulps of a midpoint
    between two bf16 neighbours: there either neighbour is accepted (an fp32
    computation with relative error e can land on either side when the
    exact value is within 256 * e ulps of the midpoint).  Zeros must carry
    the exact value's sign; NaN positions must match.  Returns how many
    elements fell in the band."""
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    exact = np.asarray(exact, dtype=np.float64)
    assert got_bits.shape == exact.shape
    got = bf16_bits_to_f64(got_bits)
    nan = np.isnan(exact)
    assert (np.isnan(got) == nan).all(), np.argwhere(np.isnan(got) != nan)[:5]
    e, g, gb = exact[~nan], got[~nan], got_bits[~nan]
    zero = e == 0
    want_zero_bits = np.where(np.signbit(e[zero]), 0x8000, 0x0000)
    assert (gb[zero] == want_zero_bits).all(), "sign of zero"
    e, g = e[~zero], g[~zero]
    assert (np.signbit(g) == np.signbit(e)).all(), "sign"
    a = np.abs(e)
    _, ex = np.frexp(a)                               # a = m * 2^ex, m in [0.5, 1)
    qe = np.maximum(ex - 8, -133)                     # bf16 quantum: 8 significant bits, subnormals 2^-133
    q = np.ldexp(a, -qe)
    lo = np.floor(q)
    frac = q - lo
    rne = np.where((frac > 0.5) | ((frac == 0.5) & (lo % 2 == 1)), lo + 1, lo)
    gq = np.ldexp(np.abs(g), -qe)
    near = np.abs(frac - 0.5) <= band
    ok = (gq == rne) | (near & ((gq == lo) | (gq == lo + 1)))
    assert ok.all(), [(float(e[i]), float(g[i])) for i in np.flatnonzero(~ok)[:5]]
    return int(near.sum())
