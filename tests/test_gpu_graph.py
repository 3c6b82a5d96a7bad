"""The fused call inside a captured HIP graph: replayed several times, with the
program's own eager work and synchronisations between replays, every replay must
equal the eager result bit for bit (the kernels use no memset nodes and the split-H
workspace needs no reset between calls)."""
import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.gpu_util import assert_parity, inputs, op, reference, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


@pytest.mark.parametrize("W,T,H,variant", [(4, 1, 2048, A.ARRMS_VARIANT_AUTO), (4, 16, 2048, A.ARRMS_VARIANT_AUTO),
                                           (8, 1, 8192, A.ARRMS_VARIANT_AUTO), (4, 128, 2048, A.ARRMS_VARIANT_SPLITH),
                                           (4, 300, 2048, A.ARRMS_VARIANT_ROW), (3, 5, 1001, A.ARRMS_VARIANT_AUTO)])
@pytest.mark.parametrize("preload", [0, 2])  # automatic, and the flat-argument twins wherever they exist
def test_graph_replays_match_eager(W, T, H, variant, preload):
    say("case graph W=%d T=%d H=%d variant=%d preload=%d" % (W, T, H, variant, preload))
    o = op()
    o.set_variant(variant)
    o.set_tuning(kernarg_preload=preload)
    try:
        cases = [inputs(W, T, H, seed=400 + i) for i in range(3)]
        xd = torch.empty((W, T, H), dtype=torch.bfloat16, device=DEV)
        rd = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        wd = torch.empty((H,), dtype=torch.bfloat16, device=DEV)
        ro = torch.empty_like(rd)
        no = torch.empty_like(rd)
        xd.copy_(cases[0][0].to(DEV)); rd.copy_(cases[0][1].to(DEV)); wd.copy_(cases[0][2].to(DEV))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            o(xd, rd, wd, 1e-6, ro, no)   # warm-up outside capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            o(xd, rd, wd, 1e-6, ro, no)
            o(xd, rd, wd, 1e-6, ro, no)   # two calls per replay: the second sees the first's workspace
        for rep in range(6):
            x, r, w = cases[rep % 3]
            xd.copy_(x.to(DEV)); rd.copy_(r.to(DEV)); wd.copy_(w.to(DEV))
            ro.fill_(0); no.fill_(0)         # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got_ro, got_no = synth.bits(ro.cpu()), synth.bits(no.cpu())
            eager_ro, eager_no = o(xd, rd, wd, 1e-6)
            torch.cuda.synchronize()
            assert np.array_equal(got_ro, synth.bits(eager_ro.cpu()))
            assert np.array_equal(got_no, synth.bits(eager_no.cpu()))
            assert_parity(got_ro, got_no, reference(x, r, w, 1e-6), "graph replay %d" % rep)
        del g
    finally:
        o.set_variant(A.ARRMS_VARIANT_AUTO)
        o.set_tuning()


@pytest.mark.parametrize("preload", [0, 2])
def test_reduce_in_graph(preload):
    say("case graph reduce preload=%d" % preload)
    x, r, w = inputs(8, 64, 5120, seed=410)
    xd = x.to(DEV)
    out = torch.empty((64, 5120), dtype=torch.bfloat16, device=DEV)
    o = op()
    o.set_tuning(kernarg_preload=preload)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            o.reduce(xd, out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            o.reduce(xd, out)
        want = reference(x, r, w, 1e-6)["reduced"]
        for rep in range(4):
            out.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(synth.bits(out.cpu()), want)
        del g
    finally:
        o.set_tuning()


@pytest.mark.parametrize("W,T,H", [(8, 16, 8192), (4, 64, 2048), (3, 5, 1001)])
def test_noalloc_in_graph(W, T, H):
    """arrms_fused_noalloc captured in a graph (split-H with its static scratch, row, and
    scalar plans): every replay, with eager work between replays, equals eager
    arrms_fused bit for bit.  The first call on the device (its one-time set-up) is made
    before capture."""
    say("case graph noalloc W=%d T=%d H=%d" % (W, T, H))
    o = op()
    cases = [inputs(W, T, H, seed=420 + i) for i in range(3)]
    xd = torch.empty((W, T, H), dtype=torch.bfloat16, device=DEV)
    rd = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    wd = torch.empty((H,), dtype=torch.bfloat16, device=DEV)
    outs = [(torch.empty_like(rd), torch.empty_like(rd)) for _ in range(2)]
    xd.copy_(cases[0][0].to(DEV)); rd.copy_(cases[0][1].to(DEV)); wd.copy_(cases[0][2].to(DEV))

    def call(k, stream):
        ro, no = outs[k]
        rc = A.arrms_fused_noalloc([xd[r].data_ptr() for r in range(W)], W, T, H, rd.data_ptr(), wd.data_ptr(),
                                   1e-6, ro.data_ptr(), no.data_ptr(), stream)
        assert rc == A.ARRMS_OK, A.arrms_status_string(rc)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0, side.cuda_stream)   # warm-up and one-time set-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream().cuda_stream
        call(0, s)
        call(1, s)   # a second call in the same replay reuses the scratch
    for rep in range(6):
        x, r, w = cases[rep % 3]
        xd.copy_(x.to(DEV)); rd.copy_(r.to(DEV)); wd.copy_(w.to(DEV))
        for ro, no in outs:
            ro.fill_(0); no.fill_(0)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager_ro, eager_no = o(xd, rd, wd, 1e-6)
        torch.cuda.synchronize()
        want_ro, want_no = synth.bits(eager_ro.cpu()), synth.bits(eager_no.cpu())
        for ro, no in outs:
            assert np.array_equal(synth.bits(ro.cpu()), want_ro)
            assert np.array_equal(synth.bits(no.cpu()), want_no)
        assert_parity(want_ro, want_no, reference(x, r, w, 1e-6), "graph noalloc replay %d" % rep)
    del g
