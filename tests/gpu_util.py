"""Helpers for the GPU parity tests: run the HIP library through the C ABI on seeded
inputs and compare with the CPU oracle element by element.

Parity bar (per element):
  residual_out : bit-identical to the oracle;
  norm_out     : within 2 BF16 steps and |err| <= 0.03125 of the oracle, NaN exactly
                 where the oracle has NaN.  The two agree bit for bit unless the
                 binary64 sums of squares (different association order) straddle a
                 binary32 rounding boundary of 1/RMS; the number of such elements
                 is returned so the tests can report it.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.bf16util import bf16_values, ulp_distance

NORM_MAX_ULP = 2
NORM_MAX_ABS = 0.03125

_op = None
# (case, norm_out elements not bit-identical, elements) of every parity check, for the summary
STATS = []


def op() -> A.FusedReduceResidualRMSNorm:
    """One handle for the whole session, with limits covering every test shape."""
    global _op
    if _op is None:
        _op = A.FusedReduceResidualRMSNorm(max_world=16, max_tokens=20000, max_hidden=65536, device=0)
    return _op


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run(x, res, w, eps, variant=A.ARRMS_VARIANT_AUTO, tuning=None, inplace=False, stream=None):
    """Run the library on CPU bf16 tensors; returns (residual_out bits, norm_out bits, plan)."""
    o = op()
    dev = torch.device("cuda", 0)
    xd, rd, wd = x.to(dev), res.to(dev), w.to(dev)
    o.set_variant(variant)
    o.set_tuning(**tuning) if tuning else o.set_tuning()
    try:
        ro = rd if inplace else torch.empty_like(rd)
        plan = o.plan(xd, rd, wd, eps, residual_out=ro)
        ro, no = o(xd, rd, wd, eps, residual_out=ro, stream=stream)
        torch.cuda.synchronize(dev)
    finally:
        o.set_variant(A.ARRMS_VARIANT_AUTO)
        o.set_tuning()
    return synth.bits(ro.cpu()), synth.bits(no.cpu()), plan


def reference(x, res, w, eps):
    return oracle.fused(synth.bits(x), synth.bits(res), synth.bits(w), eps)


def assert_parity(got_ro, got_no, ref, where="") -> int:
    """Check the parity bar; returns the count of norm_out elements not bit-identical."""
    want_ro = ref["residual_out"]
    bad = np.flatnonzero(got_ro.ravel() != want_ro.ravel())
    assert bad.size == 0, "%s: %d residual_out elements differ, first flat index %d (got %#06x want %#06x)" % (
        where, bad.size, bad[0], got_ro.ravel()[bad[0]], want_ro.ravel()[bad[0]])
    want_no = ref["norm_out"]
    gv, wv = bf16_values(got_no), bf16_values(want_no)
    gnan, wnan = np.isnan(gv), np.isnan(wv)
    assert np.array_equal(gnan, wnan), "%s: NaN positions of norm_out differ" % where
    fin = ~wnan
    if fin.any():
        d = ulp_distance(got_no[fin], want_no[fin])
        e = np.abs(gv[fin] - wv[fin])
        assert d.max() <= NORM_MAX_ULP and e.max() <= NORM_MAX_ABS, (
            "%s: norm_out off by up to %d BF16 steps / %g" % (where, int(d.max()), float(e.max())))
    n = int((got_no[fin] != want_no[fin]).sum())
    STATS.append((where, n, int(got_no.size)))
    return n


def inputs(W, T, H, seed=0, sigma=1.0, eps=1e-6, outlier_p=0.0):
    wl = synth.Workload("case", W, T, H, x_sigma=sigma, eps=eps, seed=seed, outlier_p=outlier_p)
    return synth.make_inputs(wl)
