"""Number formats: bf16, OCP E4M3 (fn), OCP E2M1 (FP4).

Test infrastructure only (see oracle/__init__.py).

Encoders are written as "pick the nearest representable value, ties to the
even code", over an explicit table of the format's non-negative finite values
(codes are monotone in value for every format here, so an even code is an
even mantissa).  Magnitudes above the largest finite value saturate to it
("satfinite"), which is what a scale or an element encoder needs when the
format has no infinity.
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------------ bf16


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact (bf16 is the top half of
    an IEEE binary32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.
    Finite inputs only (the method never feeds NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


# ------------------------------------------------------------------ E4M3 (OCP "fn")
# 1 sign, 4 exponent (bias 7), 3 mantissa.  e == 0: subnormal m * 2^-9.
# No infinities; 0x7F / 0xFF are NaN.  Largest finite: 0x7E = 448.

E4M3_MAX = 448.0


def e4m3_to_float(b: np.ndarray) -> np.ndarray:
    """E4M3 bytes -> float64 values (exact)."""
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


_E4M3_POS = e4m3_to_float(np.arange(0x7F))          # codes 0..126, increasing


def _nearest_even(table: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Index of the entry of the increasing `table` nearest to `a` (float64,
    a >= 0, a <= table[-1]); on an exact tie the even index wins."""
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - table[lo]
    dhi = table[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo)


def float_to_e4m3(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 byte: nearest, ties to even mantissa, saturating to
    +-448.  The sign is kept (also on zero)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = _nearest_even(_E4M3_POS, a).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


# ------------------------------------------------------------------ E2M1 (OCP FP4)
# 1 sign, 2 exponent (bias 1), 1 mantissa: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.

E2M1_MAX = 6.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_to_float(c: np.ndarray) -> np.ndarray:
    """4-bit codes (bit 3 = sign) -> float64."""
    c = np.asarray(c).astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def float_to_e2m1(x: np.ndarray) -> np.ndarray:
    """float -> 4-bit code: nearest of the eight magnitudes, ties to the even
    code, saturating at 6; the sign bit is copied from the input (so -0.0 and
    tiny negatives give 0x8)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    code = _nearest_even(E2M1_VALUES, a).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x8, code).astype(np.uint8)


# ------------------------------------------------------------------ nibble packing


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K] 4-bit codes -> [..., K/2] bytes; element 2j in the low nibble,
    element 2j+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
