"""arrms_fused_noalloc on the GPU, through the C ABI: the handle-free entry point whose
split-H workspace is a static device array instead of an allocation.  Its results
must equal arrms_fused's on the same inputs (same kernels, same automatic plan) and
meet the oracle parity bar; two calls in a row, the second on a smaller input, check
that what the first left in the shared scratch does not leak into the second."""
import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.gpu_util import assert_parity, inputs, op, reference, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def static_plan(W, T, H, ptrs):
    """The plan arrms_fused_noalloc takes: automatic, no tuning, the absolute limits."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    parts, res, w, ro, no = ptrs
    rc, p = A.arrms_plan(cu, A.ARRMS_VARIANT_AUTO, None, A.ARRMS_MAX_WORLD, 2 ** 31 - 1, A.ARRMS_MAX_HIDDEN,
                         parts, W, T, H, res, w, 1e-6, ro, no)
    assert rc == A.ARRMS_OK
    return p


class Case:
    """Seeded inputs on the device, with output buffers for both entry points."""

    def __init__(self, W, T, H, seed):
        self.W, self.T, self.H = W, T, H
        self.x, self.res, self.w = inputs(W, T, H, seed=seed)
        self.eps = 1e-6
        self.xd, self.rd, self.wd = self.x.to(DEV), self.res.to(DEV), self.w.to(DEV)
        self.ro = {k: torch.empty_like(self.rd) for k in ("handle", "static")}
        self.no = {k: torch.empty_like(self.rd) for k in ("handle", "static")}

    def ptrs(self, k):
        return ([self.xd[r].data_ptr() for r in range(self.W)], self.rd.data_ptr(), self.wd.data_ptr(),
                self.ro[k].data_ptr(), self.no[k].data_ptr())

    def call_static(self):
        parts, res, w, ro, no = self.ptrs("static")
        say("arrms_fused_noalloc W=%d T=%d H=%d" % (self.W, self.T, self.H))
        return A.arrms_fused_noalloc(parts, self.W, self.T, self.H, res, w, self.eps, ro, no,
                                     torch.cuda.current_stream().cuda_stream)

    def call_handle(self):
        parts, res, w, ro, no = self.ptrs("handle")
        say("arrms_fused W=%d T=%d H=%d" % (self.W, self.T, self.H))
        return A.arrms_fused(op().handle, parts, self.W, self.T, self.H, res, w, self.eps, ro, no,
                             torch.cuda.current_stream().cuda_stream)

    def check(self):
        torch.cuda.synchronize(DEV)
        bits = {k: (synth.bits(self.ro[k].cpu()), synth.bits(self.no[k].cpu())) for k in ("handle", "static")}
        assert np.array_equal(bits["static"][0], bits["handle"][0]), "residual_out differs from arrms_fused"
        assert np.array_equal(bits["static"][1], bits["handle"][1]), "norm_out differs from arrms_fused"
        ref = reference(self.x, self.res, self.w, self.eps)
        assert_parity(bits["static"][0], bits["static"][1], ref, "noalloc W=%d T=%d H=%d" % (self.W, self.T, self.H))


@pytest.mark.parametrize("big,small", [((8, 64, 8192), (8, 16, 8192)),     # split-H: the scratch is used
                                       ((4, 48, 32768), (4, 5, 32768)),    # split-H beyond the row kernels
                                       ((4, 4096, 2048), (4, 7, 2048)),    # row variant, preloaded arguments
                                       #   then one argument block: no scratch
                                       ((4, 4096, 2047), (4, 3, 2047)),    # scalar variant, likewise
                                       ((3, 300, 1001), (3, 2, 1001)),     # scalar variant: no scratch
                                       ((12, 1024, 4096), (12, 9, 4096))])  # the rank loop, then the row kernel
def test_two_calls_match_arrms_fused(big, small):
    cases = [Case(*big, seed=11), Case(*small, seed=12)]
    for c in cases:
        assert c.call_handle() == A.ARRMS_OK
    torch.cuda.synchronize(DEV)
    # two no-allocation calls back to back on the stream, the second smaller
    for c in cases:
        assert c.call_static() == A.ARRMS_OK
    for c in cases:
        c.check()


def test_split_h_cases_use_the_scratch():
    """The first two shapes above really run split-H (tokens x chunks scratch slots)."""
    for W, T, H in ((8, 64, 8192), (8, 16, 8192), (4, 48, 32768), (4, 5, 32768)):
        # disjoint fake addresses: planning compares pointers, never dereferences them
        p = static_plan(W, T, H, ([0x10000 + i * 0x10000000 for i in range(W)], 0x90000000, 0xA0000000,
                                  0xB0000000, 0xD0000000))
        assert p["variant"] == A.ARRMS_VARIANT_SPLITH and 0 < T * p["chunks_per_row"] <= A.ARRMS_NOALLOC_SCRATCH_DOUBLES


def test_scratch_limit():
    """H = 65536 at large T plans split-H with 4 chunks per row: T = 32768 fills the
    131072-slot scratch exactly and runs; T = 32769 is refused before anything is
    enqueued.  W = 1 with the partial also used as the residual (inputs may overlap);
    zero inputs give zero outputs."""
    H, T = 65536, 32768
    inp = torch.zeros((T + 1, H), dtype=torch.bfloat16, device=DEV)
    ro = torch.full((T + 1, H), 1.0, dtype=torch.bfloat16, device=DEV)
    no = torch.full((T + 1, H), 1.0, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    for t, want in ((T + 1, A.ARRMS_ERR_SCRATCH), (T, A.ARRMS_OK)):
        p = static_plan(1, t, H, ([inp.data_ptr()], inp.data_ptr(), w.data_ptr(), ro.data_ptr(), no.data_ptr()))
        assert p["variant"] == A.ARRMS_VARIANT_SPLITH and p["chunks_per_row"] == 4
        say("arrms_fused_noalloc W=1 T=%d H=%d (expect status %d)" % (t, H, want))
        rc = A.arrms_fused_noalloc([inp.data_ptr()], 1, t, H, inp.data_ptr(), w.data_ptr(), 1e-6, ro.data_ptr(),
                                   no.data_ptr(), s)
        assert rc == want, A.arrms_status_string(rc)
        torch.cuda.synchronize(DEV)
    # the accepted call wrote rows [0, T); row T was left alone
    assert int(torch.count_nonzero(ro[:T])) == 0 and int(torch.count_nonzero(no[:T])) == 0
    assert bool((ro[T] == 1).all()) and bool((no[T] == 1).all())
    del inp, ro, no
    torch.cuda.empty_cache()


def test_errors_match_arrms_fused():
    """Validation is arrms_fused's: bad sizes and aliasing are refused, T = 0 is a no-op."""
    c = Case(2, 4, 128, seed=3)
    parts, res, w, ro, no = c.ptrs("static")
    s = torch.cuda.current_stream().cuda_stream
    f = A.arrms_fused_noalloc
    assert f(parts, 2, 0, 128, res, w, 1e-6, ro, no, s) == A.ARRMS_OK
    assert f(parts, 17, 4, 128, res, w, 1e-6, ro, no, s) == A.ARRMS_ERR_INVALID_ARG
    assert f(parts, 2, 4, 65537, res, w, 1e-6, ro, no, s) == A.ARRMS_ERR_INVALID_ARG
    assert f(parts, 2, 4, 128, res, w, -1.0, ro, no, s) == A.ARRMS_ERR_INVALID_ARG
    assert f(parts, 2, 4, 128, res, w, 1e-6, ro, ro, s) == A.ARRMS_ERR_INVALID_ARG
    assert f(parts, 2, 4, 128, res, w, 1e-6, parts[1], no, s) == A.ARRMS_ERR_INVALID_ARG
    assert f(None, 2, 4, 128, res, w, 1e-6, ro, no, s) == A.ARRMS_ERR_INVALID_ARG
    torch.cuda.synchronize(DEV)


def test_torch_level_wrapper_matches_arrms_fused():
    """fused_noalloc (torch tensors, the current device) gives arrms_fused's bits."""
    c = Case(4, 77, 2048, seed=21)
    say("fused_noalloc (torch level) W=4 T=77 H=2048")
    ro, no = A.fused_noalloc(c.xd, c.rd, c.wd, c.eps, c.ro["static"], c.no["static"])
    assert ro.data_ptr() == c.ro["static"].data_ptr() and no.data_ptr() == c.no["static"].data_ptr()
    assert c.call_handle() == A.ARRMS_OK
    c.check()
