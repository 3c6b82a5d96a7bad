"""Small exact helpers for tests: BF16 bit patterns <-> Python floats and BF16 spacing.

These use only the IEEE bit layout (via ``struct``) and exact rational arithmetic;
they share nothing with the oracle or the GPU library.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np


def bf16_value(bits: int) -> float:
    """Exact value of a BF16 bit pattern (its bits are the top half of a binary32)."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def bf16_values(a: np.ndarray) -> np.ndarray:
    """float64 array of the exact values of a uint16 array of BF16 patterns."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_exact(x: float) -> int:
    """BF16 pattern of ``x``; raises if ``x`` is not exactly representable in BF16."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    if struct.unpack("<f", struct.pack("<I", u))[0] != x and not math.isnan(x):
        raise ValueError("%r is not a binary32 value" % x)
    if u & 0xFFFF:
        raise ValueError("%r is not representable in BF16" % x)
    return u >> 16


def bf16_ulp(v: float) -> Fraction:
    """Spacing of the BF16 grid at |v| (2^(e-7) on [2^e, 2^(e+1)); 2^-133 below 2^-126)."""
    a = abs(v)
    if a < 2.0 ** -126:
        return Fraction(1, 2 ** 133)
    _, e = math.frexp(a)  # a = m * 2^e with 0.5 <= m < 1, so floor(log2 a) = e - 1
    k = e - 1 - 7
    return Fraction(2) ** k


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ordinal(a) - ordinal(b)| for BF16 patterns (monotone integer map; +0 and -0 both map to 0)."""
    def ordinal(x):
        x = np.asarray(x, dtype=np.uint16).astype(np.int64)
        mag = x & 0x7FFF
        return np.where(x & 0x8000, -mag, mag)
    return np.abs(ordinal(a) - ordinal(b))
