"""Bit-exact pin of the oracle by exact rational arithmetic (tests/exact_ieee.py):
first the rounding helpers against correctly rounded library routines, then every
output bit of the oracle on seeded rows, ties, outliers, large eps and subnormals."""
import math
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.exact_ieee import BF16, BINARY32, BINARY64, check_bit_exact, round_to, sqrt_round_to


def _check(x, res, w, eps):
    check_bit_exact(oracle.default(), x, res, w, eps)


# ---------------------------------------------------------------- the helpers themselves
def test_round_to_binary32_matches_numpy_conversion():
    rng = random.Random(1)
    vals = [rng.uniform(-1, 1) * 2.0 ** rng.randint(-140, 120) for _ in range(4000)]
    vals += [1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, 2.0 ** -149 * 1.5, 2.0 ** -149 * 2.5, 2.0 ** -150]
    for d in vals:
        assert round_to(Fraction(d), BINARY32) == Fraction(float(np.float32(d))), d


def test_round_to_bf16_ties_and_subnormals():
    assert round_to(Fraction(257), BF16) == 256          # tie, even significand kept
    assert round_to(Fraction(259), BF16) == 260          # tie, rounds up to even
    assert round_to(Fraction(1) + Fraction(1, 2 ** 8), BF16) == 1
    tiny = Fraction(1, 2 ** 133)                          # BF16 subnormal quantum
    assert round_to(tiny * Fraction(3, 2), BF16) == 2 * tiny
    assert round_to(tiny / 2, BF16) == 0
    with pytest.raises(OverflowError):
        round_to(Fraction(2) ** 128, BF16)


def test_sqrt_round_to_matches_math_sqrt():
    rng = random.Random(2)
    for _ in range(4000):
        d = rng.uniform(0.5, 2.0) * 2.0 ** rng.randint(-300, 300)
        assert sqrt_round_to(Fraction(d), BINARY64) == Fraction(math.sqrt(d)), d
    for d in (4.0, 2.0, 0.25, 1e-300, 3.0):
        assert sqrt_round_to(Fraction(d), BINARY64) == Fraction(math.sqrt(d))


# ---------------------------------------------------------------- the oracle, bit for bit
def test_tiny_workload_bit_exact():
    wl = synth.WORKLOADS["tiny"]                          # W=2 T=4 H=128
    x, res, w = synth.make_inputs(wl)
    _check(synth.bits(x), synth.bits(res), synth.bits(w), wl.eps)


@pytest.mark.parametrize("W,T,H,eps,sigma,outlier_p", [
    (5, 2, 97, 1e-6, 1.0, 0.05),     # odd W and H, outliers x100
    (3, 2, 64, 0.5, 0.25, 0.0),      # eps comparable to the mean square
    (8, 1, 200, 1e-5, 30.0, 0.0),    # large values, long rank chain
    (1, 3, 40, 0.0, 1.0, 0.0),       # one rank, eps = 0
])
def test_random_rows_bit_exact(W, T, H, eps, sigma, outlier_p):
    wl = synth.Workload("exact", world=W, tokens=T, hidden=H, x_sigma=sigma, eps=eps, outlier_p=outlier_p,
                        seed=40 + W)
    x, res, w = synth.make_inputs(wl)
    _check(synth.bits(x), synth.bits(res), synth.bits(w), eps)


def test_subnormal_sums_bit_exact():
    """Partials near the bottom of the binary32 range: sums and BF16 roundings that land
    on subnormals (the rows are scaled up by the residual so that 1/RMS stays finite)."""
    rng = np.random.default_rng(3)
    W, T, H = 3, 2, 48
    x = rng.standard_normal((W, T, H)).astype(np.float32) * np.float32(2.0 ** -128)
    res = rng.standard_normal((T, H)).astype(np.float32)
    res[0, : H // 2] = 0.0                                # those elements keep the subnormal sum
    w = rng.uniform(0.5, 1.5, H).astype(np.float32)
    to_bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    _check(to_bits(x), to_bits(res), to_bits(w), 1e-6)
