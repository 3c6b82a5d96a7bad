"""GPU parity on inputs built to hit the edges of the arithmetic: exact ties of the
BF16 rounding (odd and even), subnormal sums and residuals, sums that overflow to
infinity, values near the BF16 maximum, signed zeros, and NaN / infinity inputs.
residual_out and `reduced` must equal the oracle bit for bit wherever the oracle is
not NaN, and be NaN exactly where it is (NaN payloads differ between CPU and GPU
arithmetic); norm_out is held to the usual bar."""
import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.bf16util import bf16_values, ulp_distance
from tests.gpu_util import op, reference, run, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _bits_of(values):
    return synth.bits(torch.tensor(values, dtype=torch.float32).to(torch.bfloat16))


def special_inputs(W, T, H, seed):
    """Rows of different kinds (kind = row % 6), BF16 bit patterns."""
    rng = np.random.default_rng(seed)
    x = np.zeros((W, T, H), dtype=np.uint16)
    res = np.zeros((T, H), dtype=np.uint16)
    for t in range(T):
        kind = t % 6
        if kind == 0:   # ties: x0 = v, x1 = half a BF16 step of v, the rest 0
            e = rng.integers(-20, 20, size=H)
            m = rng.integers(128, 256, size=H)
            sign = rng.choice([-1.0, 1.0], size=H)
            v = sign * m * np.exp2(e - 7.0)
            half = np.exp2(e - 8.0) * rng.choice([-1.0, 1.0], size=H)
            x[0, t] = _bits_of(v)
            x[1 % W, t] = _bits_of(half) if W > 1 else x[0, t]
            res[t] = _bits_of(np.exp2(e - 9.0) * rng.choice([-1.0, 0.0, 1.0], size=H))
        elif kind == 1:  # subnormal sums: BF16 subnormals and the smallest normals
            for r in range(W):
                x[r, t] = (rng.integers(0, 0x0100, size=H) | (rng.integers(0, 2, size=H) << 15)).astype(np.uint16)
            res[t] = (rng.integers(0, 0x0080, size=H) | (rng.integers(0, 2, size=H) << 15)).astype(np.uint16)
        elif kind == 2:  # near the BF16 maximum: sums overflow to +-inf
            for r in range(W):
                x[r, t] = (rng.integers(0x7F00, 0x7F80, size=H) | (rng.integers(0, 2, size=H) << 15)).astype(np.uint16)
            res[t] = rng.integers(0x7F00, 0x7F80, size=H).astype(np.uint16)
        elif kind == 3:  # any finite pattern, whole exponent range
            for r in range(W):
                p = rng.integers(0, 0x10000, size=H).astype(np.uint16)
                p[(p & 0x7F80) == 0x7F80] &= 0xBFFF  # clear an all-ones exponent
                x[r, t] = p
            res[t] = rng.integers(0, 0x7F00, size=H).astype(np.uint16)
        elif kind == 4:  # signed zeros and exact cancellations
            v = _bits_of(rng.integers(-4, 5, size=H).astype(np.float64))
            x[0, t] = v
            x[1 % W, t] = v ^ 0x8000 if W > 1 else v
            res[t] = rng.choice(np.array([0x0000, 0x8000], dtype=np.uint16), size=H)
        else:            # NaN and infinities among ordinary values
            for r in range(W):
                x[r, t] = _bits_of(rng.standard_normal(H))
            idx = rng.integers(0, H, size=3)
            x[0, t, idx[0]] = 0x7FC1
            x[W - 1, t, idx[1]] = 0xFF80
            res[t, idx[2]] = 0x7F80
    w = _bits_of(rng.uniform(0.5, 1.5, size=H))
    return synth.from_bits(x), synth.from_bits(res), synth.from_bits(w)


def check(got, want, what):
    gv, wv = bf16_values(got), bf16_values(want)
    wn = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), wn), "%s: NaN positions differ" % what
    bad = np.flatnonzero((got != want) & ~wn)
    assert bad.size == 0, "%s: %d elements differ, first %d (%#06x vs %#06x)" % (
        what, bad.size, bad[0], got.ravel()[bad[0]], want.ravel()[bad[0]])


def check_norm(got, want):
    gv, wv = bf16_values(got), bf16_values(want)
    wn = np.isnan(wv)
    assert np.array_equal(np.isnan(gv), wn), "norm_out: NaN positions differ"
    fin = ~wn
    assert ulp_distance(got[fin], want[fin]).max(initial=0) <= 2
    inf = np.isinf(wv)
    assert np.array_equal(gv[inf], wv[inf])


@pytest.mark.parametrize("variant", [A.ARRMS_VARIANT_ROW, A.ARRMS_VARIANT_SPLITH, A.ARRMS_VARIANT_SCALAR])
@pytest.mark.parametrize("W,H", [(1, 2048), (2, 2048), (4, 1024), (8, 5120)])
def test_special_values_fused(variant, W, H):
    say("case special values W=%d H=%d variant=%d" % (W, H, variant))
    x, res, w = special_inputs(W, 36, H, seed=W * 100 + variant)
    for eps in (1e-6, 0.0):
        ro, no, _ = run(x, res, w, eps, variant=variant)
        ref = reference(x, res, w, eps)
        check(ro, ref["residual_out"], "residual_out eps=%g" % eps)
        check_norm(no, ref["norm_out"])


@pytest.mark.parametrize("W,H", [(2, 2048), (4, 1000), (8, 5120)])
def test_special_values_reduce(W, H):
    say("case special values reduce W=%d H=%d" % (W, H))
    x, res, w = special_inputs(W, 36, H, seed=W * 7)
    got = op().reduce(x.to(DEV))
    torch.cuda.synchronize()
    check(synth.bits(got.cpu()), reference(x, res, w, 1e-6)["reduced"], "reduced")
