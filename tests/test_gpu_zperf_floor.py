"""Performance floors that catch regressions (a lost streaming hint, a spilling
kernel, a bad plan), with wide margins so that box-to-box variance cannot trip
them: the prefill shape (W=4 T=4096 H=2048) must stream at >= 4.5 TB/s (it runs
at about 5.6 TB/s on MI355X), the same rows with H = 2044 and H = 2047 (the scalar
variant, 8- and 2-byte loads) too (about 5.5 TB/s each), and a decode call (T=1) must
take < 8 us of GPU time per back-to-back call (about 2.6-3.8 us)."""

import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _gpu_us_per_call(fn, calls):
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(20):
        fn()
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(calls):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


@pytest.mark.parametrize("T,H,floor_gbs,ceil_us", [(4096, 2048, 4500.0, None), (4096, 2044, 4500.0, None),
                                                    (4096, 2047, 4500.0, None), (1, 2048, None, 8.0)])
def test_performance_floor(T, H, floor_gbs, ceil_us):
    W = 4
    sets = 4 if T > 1 else 1  # 4 x 117 MB: more than the 256 MB Infinity Cache holds (a floor, not a measurement)
    bufs = []
    for i in range(sets):
        x = torch.randn((W, T, H), device=DEV).bfloat16()
        r = torch.randn((T, H), device=DEV).bfloat16()
        bufs.append((x, r, torch.empty_like(r), torch.empty_like(r)))
    w = torch.rand(H, device=DEV).bfloat16() + 0.5
    with A.FusedReduceResidualRMSNorm(max_world=W, max_tokens=T, max_hidden=H, device=0) as op:
        calls = [op.bind(x, r, w, 1e-6, ro, no) for x, r, ro, no in bufs]
        plan = op.plan(bufs[0][0], bufs[0][1], w, 1e-6, bufs[0][2], bufs[0][3])
        assert plan["variant"] == (A.ARRMS_VARIANT_ROW if H % 8 == 0 else A.ARRMS_VARIANT_SCALAR)
        state = {"i": 0}

        def step():
            calls[state["i"] % sets]()
            state["i"] += 1

        us = _gpu_us_per_call(step, 400 if T > 1 else 2000)
    gbs = (2 * T * H * (W + 3) + 2 * H) / (us * 1e-6) / 1e9
    say("perf floor W=%d T=%d H=%d: %.2f us per call, %.0f GB/s" % (W, T, H, us, gbs))
    if floor_gbs is not None:
        assert gbs >= floor_gbs, "%.0f GB/s is below the %.0f GB/s floor" % (gbs, floor_gbs)
    if ceil_us is not None:
        assert us < ceil_us, "%.2f us per call is above %.1f us" % (us, ceil_us)
