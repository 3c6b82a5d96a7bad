"""Exact IEEE emulation of the operation, for bit-exact pins of the oracle.

Every step of the operation (page "[TLERaw] Add NVSHMEM allreduce RMSNorm tutorial",
FlagTree PR #1122, section Summary and section Implementation 3, with the rounding
readings stated in the oracle's header) is one IEEE operation in a stated format.
Here each step is carried out on exact rationals (``fractions.Fraction``) and
then rounded by ``round_to``, written from the IEEE 754 definition of round to
nearest, ties to even, for a binary format with p significand bits and minimum
normal exponent emin.  Square roots are rounded with an integer square root.
Nothing here shares code with the oracle (which works on machine floats and
integer bit patterns), so agreement on every bit of every output pins the
oracle's arithmetic, not only its error bounds.

The rounding helpers are themselves pinned against correctly rounded library
routines (numpy's binary64 -> binary32 conversion and ``math.sqrt``) in
tests/test_oracle_exact_rounding.py.
"""
import math
from fractions import Fraction

import numpy as np

from tests.bf16util import bf16_values

# (significand bits p, minimum normal exponent emin, maximum exponent emax)
BINARY64 = (53, -1022, 1023)
BINARY32 = (24, -126, 127)
BF16 = (8, -126, 127)


def _floor_log2(q: Fraction) -> int:
    """floor(log2(q)) for q > 0, exactly."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    # 2^e <= q < 2^(e+1) after at most one correction step
    if Fraction(2) ** e > q:
        e -= 1
    elif Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_to(q: Fraction, fmt) -> Fraction:
    """q rounded to the nearest value of the format, ties to the even significand.
    Subnormals use the fixed quantum 2^(emin - p + 1).  Raises OverflowError when the
    rounded magnitude reaches 2^(emax + 1) (the result would be infinite)."""
    p, emin, emax = fmt
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** (emax + 1):
        raise OverflowError("rounds to infinity")
    return sign * r


def sqrt_round_to(a: Fraction, fmt) -> Fraction:
    """sqrt(a) rounded to nearest even in the format (normal results only), for a > 0."""
    p, emin, emax = fmt
    # exponent of sqrt(a): floor(log2(sqrt(a))) = floor(floor(log2(a)) / 2)
    e = _floor_log2(a) // 2
    qe = e - p + 1
    b = a / Fraction(2) ** (2 * qe)            # sqrt(a) / 2^qe = sqrt(b)
    n = math.isqrt(b.numerator // b.denominator)  # floor(sqrt(b))
    half = Fraction(2 * n + 1, 2)
    if b > half * half or (b == half * half and n % 2 == 1):
        n += 1
    return n * Fraction(2) ** qe


def emulate(xv, rv, wv, eps):
    """The operation on exact values of BF16 inputs; returns BF16 values (as Fractions)
    of reduced, residual_out, norm_out and the binary32 1/RMS per row."""
    W, T, H = len(xv), len(rv), len(rv[0])
    f32 = lambda q: round_to(q, BINARY32)
    f64 = lambda q: round_to(q, BINARY64)
    bf = lambda q: round_to(q, BF16)
    eps32 = Fraction(float(np.float32(eps)))
    red = [[None] * H for _ in range(T)]
    ro = [[None] * H for _ in range(T)]
    nrm = [[None] * H for _ in range(T)]
    inv = [None] * T
    for t in range(T):
        ss = Fraction(0)
        for h in range(H):
            acc = xv[0][t][h]
            for r in range(1, W):
                acc = f32(acc + xv[r][t][h])
            red[t][h] = bf(acc)
            ro[t][h] = bf(f32(red[t][h] + rv[t][h]))
            ss = f64(ss + f64(ro[t][h] * ro[t][h]))
        mean = f64(ss / H)
        s = sqrt_round_to(f64(mean + eps32), BINARY64)
        inv[t] = f32(f64(1 / s))
        for h in range(H):
            nrm[t][h] = bf(f32(f32(ro[t][h] * inv[t]) * wv[h]))
    return red, ro, nrm, inv


def _fractions(a):
    return [[Fraction(float(v)) for v in row] for row in np.atleast_2d(a)]


def check_bit_exact(orc, x, res, w, eps):
    """Run the oracle ``orc`` on BF16 bit patterns and compare every output bit with the
    exact emulation (AssertionError on the first difference)."""
    out = orc.fused(x, res, w, eps)
    xv = [_fractions(bf16_values(x[r])) for r in range(x.shape[0])]
    rv = _fractions(bf16_values(res))
    wv = [Fraction(float(v)) for v in bf16_values(w)]
    red, ro, nrm, inv = emulate(xv, rv, wv, eps)
    T, H = res.shape
    for name, want in (("reduced", red), ("residual_out", ro), ("norm_out", nrm)):
        got = bf16_values(out[name])
        for t in range(T):
            for h in range(H):
                assert Fraction(float(got[t, h])) == want[t][h], (name, t, h, float(got[t, h]), float(want[t][h]))
    for t in range(T):
        assert Fraction(float(out["inv_rms"][t])) == inv[t], (t, float(out["inv_rms"][t]), float(inv[t]))
