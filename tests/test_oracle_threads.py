"""The oracle's row-split host threading (used only to time it on all host cores) gives
the same bits as one thread: rows are independent, so splitting the row range cannot
change any output."""
import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("threads", [2, 3, 8, 64])
def test_threaded_oracle_matches_single_thread(threads):
    wl = synth.Workload("threads", world=3, tokens=37, hidden=136, seed=5)
    x, res, w = synth.make_inputs(wl)
    xb, rb, wb = synth.bits(x), synth.bits(res), synth.bits(w)
    one = oracle.fused(xb, rb, wb, wl.eps)
    many = oracle.fused(xb, rb, wb, wl.eps, threads=threads)
    for k in ("reduced", "residual_out", "norm_out"):
        assert np.array_equal(one[k], many[k]), k
    assert np.array_equal(one["inv_rms"].view(np.uint32), many["inv_rms"].view(np.uint32))


def test_threaded_oracle_respects_the_row_range():
    wl = synth.Workload("threads", world=2, tokens=20, hidden=64, seed=6)
    x, res, w = synth.make_inputs(wl)
    xb, rb, wb = synth.bits(x), synth.bits(res), synth.bits(w)
    full = oracle.fused(xb, rb, wb, wl.eps)
    part = oracle.fused(xb, rb, wb, wl.eps, rows=(3, 17), threads=4)
    assert np.array_equal(part["norm_out"][3:17], full["norm_out"][3:17])
    assert not part["norm_out"][:3].any() and not part["norm_out"][17:].any()
