"""Tensors of more than 2^31 elements (4 GiB and more of BF16 each): the row, split-H,
scalar and rank-sum kernels index them with 64-bit offsets.  Inputs are zero except a few
seeded rows (the first, a middle one, the last); those rows are compared with the
oracle and every other output element must be zero (zero inputs give zero
residual_out and, with eps > 0, zero norm_out and zero reduced)."""
import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.gpu_util import assert_parity, inputs, reference, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def _sparse_inputs(W, T, H, seed):
    rows = [0, T // 2 + 1, T - 1]
    xs, rs, ws = inputs(W, len(rows), H, seed=seed)
    x = torch.zeros((W, T, H), dtype=torch.bfloat16, device=DEV)
    res = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    for i, r in enumerate(rows):
        x[:, r] = xs[:, i].to(DEV)
        res[r] = rs[i].to(DEV)
    return rows, xs, rs, ws, x, res


@pytest.mark.parametrize("W,T,H,variant", [(1, 131073, 16384, A.ARRMS_VARIANT_ROW),
                                           (2, 32769, 65536, A.ARRMS_VARIANT_SPLITH),
                                           (1, 131200, 16383, A.ARRMS_VARIANT_SCALAR)])
def test_fused_beyond_2_31_elements(W, T, H, variant):
    assert T * H > 2 ** 31
    say("case largest counts W=%d T=%d H=%d (%d elements per tensor)" % (W, T, H, T * H))
    rows, xs, rs, ws, x, res = _sparse_inputs(W, T, H, seed=T + H)
    ro = torch.empty_like(res)
    no = torch.empty_like(res)
    w = ws.to(DEV)
    with A.FusedReduceResidualRMSNorm(max_world=W, max_tokens=T, max_hidden=H, device=0) as op:
        plan = op.plan(x, res, w, 1e-6, ro, no)
        assert plan["variant"] == variant, plan
        op(x, res, w, 1e-6, ro, no)
        torch.cuda.synchronize()
    ref = reference(xs, rs, ws, 1e-6)
    got_ro = np.stack([synth.bits(ro[r].cpu()) for r in rows])
    got_no = np.stack([synth.bits(no[r].cpu()) for r in rows])
    assert_parity(got_ro, got_no, ref, "largest counts H=%d sampled rows" % H)
    # everything else is zero
    for out, got in ((ro, got_ro), (no, got_no)):
        nonzero_sampled = int(np.count_nonzero(got & 0x7FFF))
        assert int(torch.count_nonzero(out)) == nonzero_sampled
    del x, res, ro, no
    torch.cuda.empty_cache()


def test_reduce_beyond_2_31_elements():
    W, T, H = 2, 131073, 16384
    assert T * H > 2 ** 31
    say("case largest counts, rank sum W=%d T=%d H=%d" % (W, T, H))
    rows, xs, rs, ws, x, res = _sparse_inputs(W, T, H, seed=7)
    del res
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    with A.FusedReduceResidualRMSNorm(max_world=W, max_tokens=T, max_hidden=H, device=0) as op:
        op.reduce(x, out)
        torch.cuda.synchronize()
    want = reference(xs, rs, ws, 1e-6)["reduced"]
    got = np.stack([synth.bits(out[r].cpu()) for r in rows])
    assert np.array_equal(got, want)
    assert int(torch.count_nonzero(out)) == int(np.count_nonzero(got & 0x7FFF))
    del x, out
    torch.cuda.empty_cache()
