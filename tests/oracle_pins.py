"""Pins of the CPU oracle against things other than itself (a library of checks).

Every ``pin_*`` function takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with what it is pinned to.
``test_oracle_pins.py`` runs them on the oracle; ``test_oracle_mutants.py`` runs
them on deliberately broken copies of the oracle's C source to show that each
plausible mistake fails at least one pin.

The operation is the contract of the page "[TLERaw] Add NVSHMEM allreduce RMSNorm
tutorial" (FlagTree PR #1122), section Summary and section Implementation 3:
reduced = sum of the W rank partials, residual_out = reduced + residual,
norm_out = RMSNorm(residual_out, weight, eps), on BF16 rows (section Correctness).

Each test below checks the oracle against one of: a library routine (torch's
BF16 conversions), hand-derived rows (tests/golden/hand_rows.txt), exact rational
arithmetic with the IEEE error bound of each rounding, or an invariant of the
mathematics (scale invariance, rank permutation on exact sums, the RMS of the
normalised row).  A dropped term, a wrong sign or index, a transposed operand or a
different rounding point fails at least one of them.
"""
from __future__ import annotations

import math
import os
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from tests.bf16util import bf16_bits_exact, bf16_ulp, bf16_value, bf16_values
from tests.exact_ieee import check_bit_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_rows.txt")


# ---------------------------------------------------------------- BF16 rounding
def _f32_from_bits(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def pin_round_bf16_matches_torch_conversion(orc):
    """Oracle's binary32 -> BF16 rounding equals torch's RNE conversion bit for bit."""
    rng = np.random.default_rng(1)
    pats = [int(u) for u in rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64)]
    # ties (dropped half exactly 0x8000) with odd and even kept parts, near-ties, overflow edge,
    # subnormals, zeros, infinities
    for kept in (0x3F80, 0x3F81, 0x4380, 0x4381, 0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x0000, 0x8000):
        for low in (0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
            pats.append((kept << 16) | low)
    pats += [0x7F800000, 0xFF800000, 0x00000001, 0x807FFFFF]
    vals = np.array(pats, dtype=np.uint32).view(np.float32)
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for u, f, r in zip(pats, vals, ref):
        got = orc.round_bf16_bits(u)
        assert orc.round_bf16(float(f)) == got or math.isnan(f)
        if math.isnan(f):
            assert (got & 0x7FFF) > 0x7F80 and (got & 0x0040), hex(u)
        else:
            assert got == int(r), (hex(u), hex(got), hex(int(r)))


def pin_round_bf16_nan_and_overflow(orc):
    for u in (0x7FC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF):
        got = orc.round_bf16_bits(u)
        assert (got & 0x7F80) == 0x7F80 and (got & 0x007F) != 0 and (got & 0x0040)
    assert orc.round_bf16_bits(0x7F7FFFFF) == 0x7F80  # largest binary32 -> +inf
    assert orc.round_bf16_bits(0x7F7F7FFF) == 0x7F7F  # just below the tie stays finite
    assert orc.round_bf16_bits(0xFF7F8000) == 0xFF80  # tie at the top, odd kept part -> -inf


def pin_widen_is_exact(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    for b in range(0, 65536, 7):
        got = orc.widen_bf16(b)
        want = float(ref[b])
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want)


# ---------------------------------------------------------------- golden rows
def _parse_golden(path):
    cases, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0]}
        elif key == "end":
            cases.append(cur)
            cur = None
        else:
            cur[key] = vals
    return cases


GOLDEN_CASES = _parse_golden(GOLDEN)


def pin_hand_derived_row(orc, case):
    W, H = int(case["W"][0]), int(case["H"][0])
    eps = float(case["eps"][0])
    row = lambda k: np.array([bf16_bits_exact(float(v)) for v in case[k]], dtype=np.uint16)
    x = np.stack([row("x%d" % r) for r in range(W)])[:, None, :]
    res = row("residual")[None, :]
    w = row("weight")
    assert x.shape == (W, 1, H)
    out = orc.fused(x, res, w, eps)
    if "expect_residual_out" in case:
        want = bf16_values(row("expect_residual_out"))
        np.testing.assert_array_equal(bf16_values(out["residual_out"][0]), want)
    if "expect_norm_out" in case:
        want = bf16_values(row("expect_norm_out"))
        np.testing.assert_array_equal(bf16_values(out["norm_out"][0]), want)
    if "expect_inv" in case:
        assert out["inv_rms"][0] == np.float32(float(case["expect_inv"][0]))


# ---------------------------------------------------------------- special cases
def _inputs(W, T, H, seed=0, sigma=1.0):
    wl = synth.Workload("t", W, T, H, x_sigma=sigma, seed=seed)
    x, res, w = synth.make_inputs(wl)
    return synth.bits(x), synth.bits(res), synth.bits(w)


def pin_world_one_is_residual_add_plus_rmsnorm(orc):
    """W=1: reduced is x_0 itself; the op is a plain residual add followed by RMSNorm.

    The residual add is checked against torch's BF16 add (binary32 sum, one RNE),
    RMSNorm against torch's rms_norm in float64 within the rounding bound.
    """
    x, res, w = _inputs(1, 8, 256, seed=3)
    out = orc.fused(x, res, w, 1e-6)
    np.testing.assert_array_equal(out["reduced"], x[0])
    xt = synth.from_bits(x[0]).float()
    rt = synth.from_bits(res).float()
    ro_ref = synth.bits((xt + rt).to(torch.bfloat16))
    np.testing.assert_array_equal(out["residual_out"], ro_ref)
    ro64 = torch.from_numpy(bf16_values(out["residual_out"]))
    w64 = torch.from_numpy(bf16_values(w))
    ref = torch.nn.functional.rms_norm(ro64, (256,), w64, eps=float(np.float32(1e-6))).numpy()
    got = bf16_values(out["norm_out"])
    ulp = np.array([float(bf16_ulp(v)) for v in ref.ravel()]).reshape(ref.shape)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp + 4 * 2.0 ** -24 * np.abs(ref))


def pin_zero_partials(orc):
    _, res, w = _inputs(1, 6, 128, seed=4)
    x = np.zeros((3, 6, 128), dtype=np.uint16)
    out = orc.fused(x, res, w, 1e-6)
    np.testing.assert_array_equal(bf16_values(out["residual_out"]), bf16_values(res))
    ref_norm = orc.fused(res[None], np.zeros_like(res), w, 1e-6)["norm_out"]
    np.testing.assert_array_equal(out["norm_out"], ref_norm)


def pin_zero_row_zero_eps_is_nan(orc):
    """0 / sqrt(0 + 0): 0 * inf is NaN, on every element of the row."""
    x = np.zeros((2, 1, 16), dtype=np.uint16)
    w = np.full(16, bf16_bits_exact(1.0), dtype=np.uint16)
    out = orc.fused(x, np.zeros((1, 16), dtype=np.uint16), w, 0.0)
    assert np.all(np.isnan(bf16_values(out["norm_out"])))
    assert math.isinf(float(out["inv_rms"][0]))


# ---------------------------------------------------------------- exact arithmetic bounds
def _check_against_exact(x, res, w, eps, out):
    """Every output against exact rational arithmetic, within the error of its roundings.

    reduced: W-1 binary32 additions (each off by at most 2^-24 of the running sum's
    magnitude) and one BF16 rounding (half a BF16 spacing).  residual_out: one binary32
    addition and one BF16 rounding.  norm_out: the exact real ro*w/sqrt(mean(ro^2)+eps),
    off by at most 4*2^-24 relative (1/RMS rounded to binary32 plus two binary32
    products) and half a BF16 spacing.
    """
    W, T, H = x.shape
    getcontext().prec = 50
    xv = [bf16_values(x[r]) for r in range(W)]
    rv = bf16_values(res)
    wv = bf16_values(w)
    red = bf16_values(out["reduced"])
    ro = bf16_values(out["residual_out"])
    nv = bf16_values(out["norm_out"])
    eps_exact = Decimal(float(np.float32(eps)))
    for t in range(T):
        ss = Fraction(0)
        for h in range(H):
            partial, run_max = Fraction(0), Fraction(0)
            for r in range(W):
                partial += Fraction(xv[r][t, h])
                run_max = max(run_max, abs(partial))
            got = Fraction(red[t, h])
            bound = bf16_ulp(red[t, h]) / 2 + (W - 1) * run_max / 2 ** 24
            assert abs(got - partial) <= bound, (t, h)
            s = Fraction(red[t, h]) + Fraction(rv[t, h])
            assert abs(Fraction(ro[t, h]) - s) <= bf16_ulp(ro[t, h]) / 2 + abs(s) / 2 ** 24, (t, h)
            ss += Fraction(ro[t, h]) ** 2
        denom = (Decimal(ss.numerator) / Decimal(ss.denominator) / H + eps_exact).sqrt()
        for h in range(H):
            exact = Decimal(ro[t, h]) * Decimal(wv[h]) / denom
            err = abs(Decimal(nv[t, h]) - exact)
            tol = Decimal(float(bf16_ulp(float(exact)))) / 2 + abs(exact) * Decimal(4) / Decimal(2 ** 24)
            assert err <= tol, (t, h, float(err), float(tol))


def pin_tiny_workload_exact_bounds(orc):
    """W=2, T=4, H=128 (the tiny parity workload), every element against exact arithmetic."""
    wl = synth.WORKLOADS["tiny"]
    x, res, w = synth.make_inputs(wl)
    x, res, w = synth.bits(x), synth.bits(res), synth.bits(w)
    _check_against_exact(x, res, w, wl.eps, orc.fused(x, res, w, wl.eps))


def pin_random_rows_exact_bounds(orc, W, H, eps, sigma):
    """Mixed W, non-power-of-two H, eps comparable to the mean square, large values."""
    x, res, w = _inputs(W, 3, H, seed=11 + W, sigma=sigma)
    _check_against_exact(x, res, w, eps, orc.fused(x, res, w, eps))


# ---------------------------------------------------------------- invariants
def pin_rms_of_normalised_row_is_one(orc):
    """sqrt(mean((norm_out / weight)^2)) = 1 up to BF16 rounding when mean square >> eps."""
    wl = synth.WORKLOADS["decode_t16"]
    x, res, w = synth.make_inputs(wl)
    out = orc.fused(synth.bits(x), synth.bits(res), synth.bits(w), wl.eps)
    ratio = bf16_values(out["norm_out"]) / bf16_values(synth.bits(w))[None, :]
    rms = np.sqrt(np.mean(ratio * ratio, axis=1))
    assert np.all(np.abs(rms - 1.0) <= 2.0 ** -8)


def pin_rms_with_large_eps(orc):
    """With eps comparable to the mean square, RMS(norm/weight) = sqrt(m / (m + eps))."""
    x, res, w = _inputs(2, 4, 512, seed=5, sigma=0.1)
    eps = 0.02
    out = orc.fused(x, res, w, eps)
    ro = bf16_values(out["residual_out"])
    m = np.mean(ro * ro, axis=1)
    ratio = bf16_values(out["norm_out"]) / bf16_values(w)[None, :]
    rms = np.sqrt(np.mean(ratio * ratio, axis=1))
    np.testing.assert_allclose(rms, np.sqrt(m / (m + float(np.float32(eps)))), rtol=2.0 ** -8)


def pin_power_of_two_scaling(orc, k):
    """eps = 0: scaling partials and residual by 2^k scales residual_out by exactly 2^k and
    leaves norm_out bit-identical (every rounding commutes with an exact power-of-two scale)."""
    x, res, w = _inputs(4, 5, 256, seed=6)
    scale = lambda a: synth.bits((synth.from_bits(a).double() * 2.0 ** k).to(torch.bfloat16))
    xs, rs = scale(x), scale(res)
    assert np.array_equal(bf16_values(xs), bf16_values(x) * 2.0 ** k)  # exact scaling, no overflow
    a = orc.fused(x, res, w, 0.0)
    b = orc.fused(xs, rs, w, 0.0)
    np.testing.assert_array_equal(bf16_values(b["residual_out"]), bf16_values(a["residual_out"]) * 2.0 ** k)
    np.testing.assert_array_equal(b["norm_out"], a["norm_out"])


def pin_rank_permutation_exact_sums(orc):
    """Small-integer partials: every binary32 sum is exact, so any rank order gives the
    same bits, and reduced equals the integer sum (brute force in Python ints)."""
    rng = np.random.default_rng(7)
    W, T, H = 5, 3, 64
    ints = rng.integers(-8, 9, size=(W, T, H))
    x = np.vectorize(lambda v: bf16_bits_exact(float(v)), otypes=[np.uint16])(ints)
    _, res, w = _inputs(1, T, H, seed=8)
    base = orc.fused(x, res, w, 1e-6)
    np.testing.assert_array_equal(bf16_values(base["reduced"]), ints.sum(axis=0).astype(np.float64))
    for perm in ([4, 3, 2, 1, 0], [2, 0, 4, 1, 3]):
        other = orc.fused(x[perm], res, w, 1e-6)
        for k in ("reduced", "residual_out", "norm_out"):
            np.testing.assert_array_equal(other[k], base[k])


def pin_row_range_and_determinism(orc):
    x, res, w = _inputs(3, 9, 96, seed=9)
    full = orc.fused(x, res, w, 1e-6)
    again = orc.fused(x, res, w, 1e-6)
    part = orc.fused(x, res, w, 1e-6, rows=(2, 7))
    for k in ("reduced", "residual_out", "norm_out"):
        np.testing.assert_array_equal(full[k], again[k])
        np.testing.assert_array_equal(part[k][2:7], full[k][2:7])
        assert not part[k][:2].any() and not part[k][7:].any()


def pin_rows_are_independent(orc):
    """Each token row depends only on its own inputs: permuting rows permutes outputs."""
    x, res, w = _inputs(2, 6, 64, seed=10)
    perm = [5, 3, 0, 1, 4, 2]
    a = orc.fused(x, res, w, 1e-6)
    b = orc.fused(x[:, perm], res[perm], w, 1e-6)
    for k in ("residual_out", "norm_out"):
        np.testing.assert_array_equal(b[k], a[k][perm])


def _nearest_f32(exact: Decimal) -> np.float32:
    """binary32 nearest to a positive Decimal (ties cannot occur for these irrational values)."""
    c = np.float32(float(exact))
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda f: abs(Decimal(float(f)) - exact))


def pin_inv_rms_is_correctly_rounded(orc):
    """1/RMS is 1/sqrt(mean(ro^2) + eps) of the exact BF16 residual_out values, rounded once
    to binary32.  A binary32 sum of squares, a sum instead of a mean, or eps outside the root
    misses it on most rows."""
    getcontext().prec = 60
    for W, T, H, eps, seed in ((4, 12, 2048, 1e-6, 21), (2, 12, 5120, 1e-5, 22), (8, 6, 1000, 0.25, 23)):
        x, res, w = _inputs(W, T, H, seed=seed)
        out = orc.fused(x, res, w, eps)
        ro = bf16_values(out["residual_out"])
        for t in range(T):
            ss = sum(Fraction(v) ** 2 for v in ro[t])
            m = Decimal(ss.numerator) / Decimal(ss.denominator) / Decimal(H)
            exact = Decimal(1) / (m + Decimal(float(np.float32(eps)))).sqrt()
            assert out["inv_rms"][t] == _nearest_f32(exact), (W, H, t)


def pin_exact_emulation(orc, W, T, H, eps, sigma, outlier_p):
    """Every output bit equals an exact rational emulation of the IEEE steps."""
    wl = synth.Workload("exact", world=W, tokens=T, hidden=H, x_sigma=sigma, eps=eps, outlier_p=outlier_p,
                        seed=70 + W)
    x, res, w = synth.make_inputs(wl)
    check_bit_exact(orc, synth.bits(x), synth.bits(res), synth.bits(w), eps)


def _bf16_rne_f32(a: np.ndarray) -> np.ndarray:
    """Input search helper: binary32 array rounded to BF16 (as binary32), nearest even."""
    u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def pin_exact_emulation_order_sensitive_rows(orc):
    """Rows where the order of the two final products matters after BF16 rounding.

    (ro * inv) * w and (ro * w) * inv differ in one binary32 ulp now and then, which
    BF16 rounding almost always hides; random workloads rarely expose the order.
    Rows are searched (seeded, in numpy binary32) where the two orders give different
    BF16 values, then the oracle is checked bit for bit against the exact emulation on
    them (W=1 and a zero residual, so residual_out is the searched row itself)."""
    rng = np.random.default_rng(123)
    T, H, eps = 1 << 18, 16, 1e-6  # about 8 such elements expected per million
    ro = _bf16_rne_f32(rng.standard_normal((T, H)).astype(np.float32))
    w = _bf16_rne_f32(rng.uniform(0.5, 1.5, H).astype(np.float32))
    ss = np.cumsum(ro.astype(np.float64) ** 2, axis=1)[:, -1]          # sequential in h
    inv = (1.0 / np.sqrt(ss / H + float(np.float32(eps)))).astype(np.float32)[:, None]
    a = _bf16_rne_f32((ro * inv).astype(np.float32) * w)
    b = _bf16_rne_f32((ro * w).astype(np.float32) * inv)
    rows = np.nonzero((a != b).any(axis=1))[0][:6]
    assert len(rows) >= 3, "search found too few order-sensitive rows"
    to_bits = lambda v: (np.ascontiguousarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = to_bits(ro[rows])[None]
    check_bit_exact(orc, x, np.zeros((len(rows), H), dtype=np.uint16), to_bits(w), eps)


PINS = [
    ("round_bf16_vs_torch", pin_round_bf16_matches_torch_conversion, {}),
    ("round_bf16_nan_overflow", pin_round_bf16_nan_and_overflow, {}),
    ("widen_exact", pin_widen_is_exact, {}),
    *[("golden_" + c["name"], pin_hand_derived_row, {"case": c}) for c in GOLDEN_CASES],
    ("world_one", pin_world_one_is_residual_add_plus_rmsnorm, {}),
    ("zero_partials", pin_zero_partials, {}),
    ("zero_row_zero_eps_nan", pin_zero_row_zero_eps_is_nan, {}),
    ("tiny_exact_bounds", pin_tiny_workload_exact_bounds, {}),
    *[("random_exact_bounds_W%d_H%d" % (W, H), pin_random_rows_exact_bounds,
       {"W": W, "H": H, "eps": eps, "sigma": sg})
      for W, H, eps, sg in [(4, 64, 1e-6, 1.0), (8, 40, 0.5, 0.05), (3, 24, 1e-5, 100.0)]],
    ("inv_rms_correctly_rounded", pin_inv_rms_is_correctly_rounded, {}),
    ("rms_is_one", pin_rms_of_normalised_row_is_one, {}),
    ("rms_large_eps", pin_rms_with_large_eps, {}),
    *[("pow2_scaling_%d" % k, pin_power_of_two_scaling, {"k": k}) for k in (3, -3, 10)],
    ("rank_permutation_exact", pin_rank_permutation_exact_sums, {}),
    ("row_range_determinism", pin_row_range_and_determinism, {}),
    ("rows_independent", pin_rows_are_independent, {}),
    *[("exact_emulation_W%d_H%d" % (W, H), pin_exact_emulation,
       {"W": W, "T": T, "H": H, "eps": eps, "sigma": sg, "outlier_p": op})
      for W, T, H, eps, sg, op in [(2, 4, 128, 1e-6, 1.0, 0.0), (5, 2, 72, 1e-6, 1.0, 0.05),
                                   (3, 2, 40, 0.5, 0.25, 0.0)]],
    ("exact_emulation_order_sensitive", pin_exact_emulation_order_sensitive_rows, {}),
]
