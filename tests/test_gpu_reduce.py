"""GPU parity of the rank sum alone (arrms_reduce) and of the page's two-stage form
(rank sum, then the residual + RMSNorm epilogue as arrms_fused with W=1) against the
CPU oracle's `reduced`, `residual_out` and `norm_out`."""
import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.gpu_util import assert_parity, inputs, op, reference, run, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def reduce_gpu(x, reduced=None):
    o = op()
    xd = x.to(DEV)
    out = o.reduce(xd, reduced)
    torch.cuda.synchronize()
    return synth.bits(out.cpu())


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8, 9, 16])
@pytest.mark.parametrize("T,H", [(1, 8), (3, 3), (5, 1001), (37, 2048), (4096, 2048), (7, 5120)])
def test_reduce_matches_oracle(W, T, H):
    say("case reduce W=%d T=%d H=%d" % (W, T, H))
    x, res, w = inputs(W, T, H, seed=300 + W + T, outlier_p=0.01)
    got = reduce_gpu(x)
    want = reference(x, res, w, 1e-6)["reduced"]
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, "%d reduced elements differ" % bad.size


def test_reduce_full_size_ragged_outliers():
    wl = synth.WORKLOADS["ragged_outliers"]
    say("case reduce full size %s" % wl.name)
    x, res, w = synth.make_inputs(wl)
    got = reduce_gpu(x)
    want = reference(x, res, w, wl.eps)["reduced"]
    assert np.array_equal(got, want)


def test_reduce_in_place_into_a_partial():
    say("case reduce in place")
    x, res, w = inputs(4, 33, 2048, seed=301)
    xd = x.to(DEV)
    out = op().reduce(xd, reduced=xd[2])
    torch.cuda.synchronize()
    assert np.array_equal(synth.bits(out.cpu()), reference(x, res, w, 1e-6)["reduced"])


def _placed(t, off_bytes):
    """A GPU copy of CPU tensor t whose data starts off_bytes after a 256-byte boundary."""
    n = t.numel()
    buf = torch.zeros(n + 256, dtype=torch.bfloat16, device=DEV)
    base = (-buf.data_ptr()) % 256 // 2
    view = buf[base + off_bytes // 2: base + off_bytes // 2 + n].view(t.shape)
    view.copy_(t.to(DEV))
    assert view.data_ptr() % 256 == off_bytes
    return view


# The rank sum is flat over T*H elements: with every tensor at the same offset it
# loads 16 bytes at a time after a head of up to 7 elements; where the offsets differ
# it takes the widest load at which they agree (8, 4 or 2 bytes).
@pytest.mark.parametrize("W,T,H,part_off,out_off,elems", [
    (3, 11, 2048, 2, 2, 8), (3, 11, 2048, 14, 14, 8), (4, 64, 1000, 8, 8, 8), (2, 4096, 2048, 6, 6, 8),
    (4, 33, 2048, 0, 8, 4), (4, 33, 2048, 0, 4, 2), (4, 33, 2048, 0, 2, 1), (4, 33, 2047, 8, 0, 4),
    (1, 1, 3, 2, 2, 8), (1, 1, 5, 0, 4, 2), (2, 3, 5, 0, 6, 1), (16, 7, 999, 6, 6, 8), (9, 5, 2049, 0, 12, 2), (12, 300, 1000, 4, 0, 2),
    (8, 513, 5120, 2, 0, 1),
])
def test_reduce_at_offsets(W, T, H, part_off, out_off, elems):
    say("case reduce offsets W=%d T=%d H=%d partials +%d out +%d" % (W, T, H, part_off, out_off))
    x, res, w = inputs(W, T, H, seed=302 + W + T + part_off + out_off, outlier_p=0.01)
    parts = [_placed(x[r], part_off) for r in range(W)]
    out = _placed(torch.zeros(T, H, dtype=torch.bfloat16), out_off)
    rc, plan = A.arrms_plan_reduce(256, None, 16, 20000, 65536, [p.data_ptr() for p in parts], W, T, H,
                                   out.data_ptr())
    assert rc == A.ARRMS_OK and plan["elems_per_load"] == elems
    assert plan["variant"] == (A.ARRMS_VARIANT_REDUCE if elems == 8 else A.ARRMS_VARIANT_REDUCE_SCALAR)
    op().reduce(parts, out)
    torch.cuda.synchronize()
    assert np.array_equal(synth.bits(out.cpu()), reference(x, res, w, 1e-6)["reduced"])


@pytest.mark.parametrize("off", [0, 6])
def test_reduce_in_place_at_an_offset(off):
    say("case reduce in place at +%d" % off)
    W, T, H = 4, 17, 1003
    x, res, w = inputs(W, T, H, seed=305 + off)
    parts = [_placed(x[r], off) for r in range(W)]
    out = op().reduce(parts, reduced=parts[1])
    torch.cuda.synchronize()
    assert np.array_equal(synth.bits(out.cpu()), reference(x, res, w, 1e-6)["reduced"])


@pytest.mark.parametrize("elems", [1, 2, 4])
@pytest.mark.parametrize("W", [3, 8, 11])
def test_reduce_tuned_load_widths(elems, W):
    """Tuning caps the load width: the same aligned tensors through 2-, 4- and 8-byte loads."""
    say("case reduce width %d W=%d" % (elems, W))
    x, res, w = inputs(W, 129, 1000, seed=320 + W + elems)
    o = op()
    o.set_tuning(scalar_elems=elems)
    try:
        got = reduce_gpu(x)
    finally:
        o.set_tuning()
    assert np.array_equal(got, reference(x, res, w, 1e-6)["reduced"])


@pytest.mark.parametrize("W,T,H", [(4, 4096, 2048), (8, 129, 5120), (2, 4, 128)])
def test_two_stage_form_equals_fused(W, T, H):
    """Rank sum, then the epilogue as a one-rank fused call: the same bits as one fused call."""
    say("case two-stage W=%d T=%d H=%d" % (W, T, H))
    x, res, w = inputs(W, T, H, seed=303 + T)
    o = op()
    xd, rd, wd = x.to(DEV), res.to(DEV), w.to(DEV)
    red = o.reduce(xd)
    ro2, no2 = o([red], rd, wd, 1e-6)
    ro1, no1 = o(xd, rd, wd, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(ro1.view(torch.int16), ro2.view(torch.int16))
    assert torch.equal(no1.view(torch.int16), no2.view(torch.int16))
    assert_parity(synth.bits(ro2.cpu()), synth.bits(no2.cpu()), reference(x, res, w, 1e-6), "two-stage")


@pytest.mark.parametrize("W", [2, 4, 8, 12])
@pytest.mark.parametrize("vpt", [1, 2, 4])
@pytest.mark.parametrize("k", [0, 3, 64])
def test_reduce_tunings(W, vpt, k):
    """Every rank-sum kernel instance and XCD mapping, on a ragged element count."""
    if W > 8 and vpt > 1:
        pytest.skip("W > 8 has only the one-vector instance")
    say("case reduce tuning W=%d vpt=%d K=%d" % (W, vpt, k))
    x, res, w = inputs(W, 301, 1000, seed=310 + W)
    o = op()
    o.set_tuning(vec_per_thread=vpt, xcd_chunk=k)
    try:
        got = reduce_gpu(x)
    finally:
        o.set_tuning()
    assert np.array_equal(got, reference(x, res, w, 1e-6)["reduced"])


# Rank-sum kernels with preloaded arguments (the flat-argument twins) and with one
# argument block, each forced: every load width (tuned narrower on aligned tensors),
# 1, 2 and 4 vectors per lane, a head and tail from an offset, W = 1..8.
@pytest.mark.parametrize("W,vpt,elems,off", [(1, 1, 8, 0), (2, 2, 8, 0), (4, 4, 8, 0), (5, 0, 4, 0), (6, 0, 2, 0),
                                             (8, 0, 1, 0), (3, 1, 8, 6), (7, 2, 8, 2)])
@pytest.mark.parametrize("preload", [1, 2])
def test_reduce_kernarg_preload_paths(W, vpt, elems, off, preload):
    T, H = 301, 1000
    say("case reduce preload=%d W=%d vpt=%d elems=%d +%d" % (preload, W, vpt, elems, off))
    x, res, w = inputs(W, T, H, seed=330 + W + elems + preload)
    parts = [_placed(x[r], off) for r in range(W)]
    out = _placed(torch.zeros(T, H, dtype=torch.bfloat16), off)
    tun = dict(kernarg_preload=preload, vec_per_thread=vpt, scalar_elems=elems if elems < 8 else 0)
    rc, plan = A.arrms_plan_reduce(256, A.arrms_tuning_t.make(**tun), 16, 20000, 65536,
                                   [p.data_ptr() for p in parts], W, T, H, out.data_ptr())
    assert rc == A.ARRMS_OK and plan["kernarg_preload"] == (preload == 2) and plan["elems_per_load"] == elems, plan
    o = op()
    o.set_tuning(**tun)
    try:
        o.reduce(parts, out)
        torch.cuda.synchronize()
    finally:
        o.set_tuning()
    assert np.array_equal(synth.bits(out.cpu()), reference(x, res, w, 1e-6)["reduced"])
