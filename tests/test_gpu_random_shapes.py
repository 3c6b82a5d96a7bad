"""Seeded random cases against the oracle: world sizes, token counts, hidden sizes
(multiples of 8 and not), forced variants, tensors placed at 2-, 4-, 8-, 12- and
16-byte offsets (16-byte vector paths and every scalar load width), in-place residual,
kernels with preloaded arguments forced in every other case, and the rank sum alone.  Every element is compared, to the parity bar of
tests/gpu_util.py."""
import os

import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.gpu_util import assert_parity, inputs, op, reference, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
VNAMES = {A.ARRMS_VARIANT_AUTO: "auto", A.ARRMS_VARIANT_ROW: "row", A.ARRMS_VARIANT_SPLITH: "splith",
          A.ARRMS_VARIANT_SCALAR: "scalar"}


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        W = int(rng.integers(1, 17))
        T = int(rng.integers(1, 260))
        H = int(rng.integers(1, 9000)) if rng.random() < 0.25 else 8 * int(rng.integers(1, 1025))
        # byte offset of each tensor from a 256-byte boundary (partials, residual, weight,
        # residual_out, norm_out): all 16-byte aligned in 70 % of the cases, else one or two
        # tensors at a 2-, 4-, 8-, 12- or 18-byte offset (every load width of the scalar kernel)
        offs = [16 * int(rng.integers(0, 2)) for _ in range(W + 4)]
        if rng.random() >= 0.7:
            for k in rng.choice(W + 4, size=int(rng.integers(1, 3)), replace=False):
                offs[int(k)] = int(rng.choice([2, 4, 8, 12, 18]))
        inplace = bool(rng.random() < 0.25)
        if inplace:
            offs[W + 2] = offs[W]
        vector_ok = H % 8 == 0 and all(o % 16 == 0 for o in offs)
        choices = [A.ARRMS_VARIANT_AUTO, A.ARRMS_VARIANT_SCALAR]
        if vector_ok:
            # the row kernels hold a row in registers: up to 16384 elements for W <= 8, 4096 above
            row_ok = H <= (A.ARRMS_ROW_MAX_HIDDEN if W <= 8 else 4096)
            choices += [A.ARRMS_VARIANT_SPLITH] + ([A.ARRMS_VARIANT_ROW] if row_ok else [])
        variant = int(rng.choice(choices))
        out.append((i, W, T, H, tuple(offs), inplace, variant, 1000 + i))
    return out


# ARRMS_RANDOM_CASES / ARRMS_RANDOM_SEED scale the sweep up for a longer stress run.
CASES = _cases(int(os.environ.get("ARRMS_RANDOM_CASES", "64")), int(os.environ.get("ARRMS_RANDOM_SEED", "2024")))


def _placed(t, off_bytes):
    """A GPU copy of t whose data starts off_bytes after a 256-byte boundary."""
    n = t.numel()
    buf = torch.zeros(n + 256, dtype=torch.bfloat16, device=DEV)
    base = (-buf.data_ptr()) % 256 // 2
    view = buf[base + off_bytes // 2: base + off_bytes // 2 + n].view(t.shape)
    view.copy_(t.to(DEV))
    assert view.data_ptr() % 256 == off_bytes
    return view


@pytest.mark.parametrize("i,W,T,H,offs,inplace,variant,seed", CASES, ids=["case%d" % c[0] for c in CASES])
def test_random_case(i, W, T, H, offs, inplace, variant, seed):
    preload = 2 if i % 2 else 0  # odd cases: the flat-argument twins wherever they exist
    where = "random case %d: W=%d T=%d H=%d offsets=%s inplace=%s variant=%s seed=%d preload=%d" % (
        i, W, T, H, offs, inplace, VNAMES[variant], seed, preload)
    say(where)
    x, res, w = inputs(W, T, H, seed=seed, outlier_p=0.01 if i % 3 == 0 else 0.0)
    xs = [_placed(x[r], offs[r]) for r in range(W)]
    rs = _placed(res, offs[W])
    ws = _placed(w, offs[W + 1])
    ro = rs if inplace else _placed(torch.zeros_like(res), offs[W + 2])
    no = _placed(torch.zeros_like(res), offs[W + 3])
    o = op()
    o.set_variant(variant)
    o.set_tuning(kernarg_preload=preload)
    try:
        plan = o.plan(xs, rs, ws, 1e-6, ro, no)
        if variant != A.ARRMS_VARIANT_AUTO:
            assert plan["variant"] == variant
        o(xs, rs, ws, 1e-6, ro, no)
        torch.cuda.synchronize()
    finally:
        o.set_variant(A.ARRMS_VARIANT_AUTO)
        o.set_tuning()
    n = assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, res, w, 1e-6), where)
    say("  plan %s, norm_out not bit-identical: %d" % (plan, n))


REDUCE_CASES = [(i, W, T, H, offs[:W] + (offs[W + 2],), 2000 + i) for i, W, T, H, offs, _, _, _ in _cases(16, 77)]


@pytest.mark.parametrize("i,W,T,H,offs,seed", REDUCE_CASES, ids=["reduce%d" % c[0] for c in REDUCE_CASES])
def test_random_reduce_case(i, W, T, H, offs, seed):
    preload = 2 if i % 2 else 0
    say("random reduce case %d: W=%d T=%d H=%d offsets=%s seed=%d preload=%d" % (i, W, T, H, offs, seed, preload))
    x, res, w = inputs(W, T, H, seed=seed)
    xs = [_placed(x[r], offs[r]) for r in range(W)]
    out = _placed(torch.zeros_like(res), offs[W])
    o = op()
    o.set_tuning(kernarg_preload=preload)
    try:
        o.reduce(xs, out)
        torch.cuda.synchronize()
    finally:
        o.set_tuning()
    want = reference(x, res, w, 1e-6)["reduced"]
    got = synth.bits(out.cpu())
    assert np.array_equal(got, want), "reduced differs in %d elements" % int((got != want).sum())
