"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on the same
seeded inputs, element by element.  See tests/gpu_util.py for the bar."""
import numpy as np
import pytest
import torch

import residual_add_rmsnorm_arrms_amd as A
import synth
from tests.bf16util import bf16_values
from tests.gpu_util import assert_parity, inputs, op, reference, run, say

pytestmark = pytest.mark.gpu

ROW, SPLITH, SCALAR, AUTO = A.ARRMS_VARIANT_ROW, A.ARRMS_VARIANT_SPLITH, A.ARRMS_VARIANT_SCALAR, A.ARRMS_VARIANT_AUTO
VNAME = {AUTO: "auto", ROW: "row", SPLITH: "splith", SCALAR: "scalar"}


def parity(W, T, H, variant=AUTO, tuning=None, seed=0, sigma=1.0, eps=1e-6, outlier_p=0.0, inplace=False):
    where = "W=%d T=%d H=%d variant=%s tuning=%s seed=%d inplace=%s" % (W, T, H, VNAME[variant], tuning, seed,
                                                                         inplace)
    say("case " + where)
    x, res, w = inputs(W, T, H, seed=seed, sigma=sigma, eps=eps, outlier_p=outlier_p)
    ro, no, plan = run(x, res, w, eps, variant=variant, tuning=tuning, inplace=inplace)
    ref = reference(x, res, w, eps)
    n = assert_parity(ro, no, ref, where)
    say("  plan %s, norm_out not bit-identical: %d of %d" % (plan, n, no.size))
    return plan, n


# ------------------------------------------------------------ named workloads
@pytest.mark.parametrize("name", ["tiny", "decode_t1", "decode_t16", "decode_t128", "prefill"])
def test_named_workload(name):
    wl = synth.WORKLOADS[name]
    say("workload %s" % name)
    x, res, w = synth.make_inputs(wl)
    ro, no, plan = run(x, res, w, wl.eps)
    n = assert_parity(ro, no, reference(x, res, w, wl.eps), name)
    say("  plan %s, norm_out not bit-identical: %d of %d" % (plan, n, no.size))


@pytest.mark.parametrize("name", ["large_hidden", "ragged_outliers"])
def test_full_size_workload(name):
    """Full-size workloads in the launch configuration the benchmark times (automatic
    variant), every element compared with the oracle."""
    wl = synth.WORKLOADS[name]
    say("workload %s (full size, all %d rows)" % (name, wl.tokens))
    x, res, w = synth.make_inputs(wl)
    ro, no, plan = run(x, res, w, wl.eps)
    ref = reference(x, res, w, wl.eps)
    n = assert_parity(ro, no, ref, name)
    say("  plan %s, norm_out not bit-identical: %d of %d" % (plan, n, no.size))


# ------------------------------------------------------------ sweeps
TOKENS = [1, 2, 3, 15, 16, 17, 63, 64, 127, 128, 255, 256, 257, 1024, 4096, 16383]


@pytest.mark.parametrize("T", TOKENS)
@pytest.mark.parametrize("variant", [AUTO, ROW, SPLITH, SCALAR])
def test_token_sweep(T, variant):
    plan, _ = parity(4, T, 2048, variant=variant, seed=T)
    if variant != AUTO:
        assert plan["variant"] == variant


HIDDEN = [8, 64, 128, 1000, 1001, 2040, 2048, 5120, 8192, 16384, 24576]


@pytest.mark.parametrize("H", HIDDEN)
@pytest.mark.parametrize("variant", [AUTO, ROW, SPLITH, SCALAR])
def test_hidden_sweep(H, variant):
    vector_ok = H % 8 == 0
    if variant == ROW and (not vector_ok or H > A.ARRMS_ROW_MAX_HIDDEN):
        pytest.skip("row variant needs H % 8 == 0 and H <= 16384")
    if variant == SPLITH and not vector_ok:
        pytest.skip("split-H variant needs H % 8 == 0")
    parity(4, 37, H, variant=variant, seed=H)


WORLDS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16]


@pytest.mark.parametrize("W", WORLDS)
@pytest.mark.parametrize("variant", [AUTO, ROW, SPLITH, SCALAR])
def test_world_sweep(W, variant):
    parity(W, 33, 2048, variant=variant, seed=100 + W)


# The scalar variant walks a row in spans of 8 * lanes elements: a row that fits one
# span of at most 1024 lanes gets just enough lanes and keeps
# residual_out in registers; a longer row runs on 256 lanes over several spans and
# re-reads it.  Single-element rows,
# rows ending one element into a new span, in place, generic W and the largest H.
SCALAR_SPANS = [(4, 5, 1, False), (3, 7, 3, False), (4, 9, 8191, False), (4, 9, 8193, True),
                (9, 6, 20001, True), (2, 3, 65535, False), (8, 3, 65536, True), (16, 2, 9000, False)]


@pytest.mark.parametrize("W,T,H,inplace", SCALAR_SPANS)
def test_scalar_spans(W, T, H, inplace):
    plan, _ = parity(W, T, H, variant=SCALAR, inplace=inplace, seed=H)
    assert plan["variant"] == SCALAR
    one_span = -(-(-(-H // 8)) // 64) * 64
    assert plan["block"] == (one_span if one_span <= 1024 else 256)


# The scalar variant loads 4, 2 or 1 BF16 elements at a time: the widest that H and
# every pointer's alignment allow.  Each width, from H and from pointer offsets (on
# every tensor, or on one tensor only), in one span and in several, at T = 1 and at
# a prefill-sized T, with the rank count specialised and generic.
SCALAR_WIDTHS = [
    # W, T, H, byte offset, which tensors, load width
    (4, 4096, 2044, 0, "all", 4), (4, 1, 2044, 0, "all", 4), (4, 4096, 5122, 0, "all", 2),
    (4, 1, 5122, 0, "all", 2), (4, 4096, 2047, 0, "all", 1), (3, 300, 2046, 0, "all", 2),
    (4, 4096, 2048, 8, "all", 4), (4, 130, 2048, 4, "all", 2), (4, 130, 2048, 2, "all", 1),
    (4, 64, 2048, 8, "residual", 4), (4, 64, 2048, 4, "weight", 2), (4, 64, 2048, 2, "partial", 1),
    (4, 64, 2044, 4, "norm_out", 2), (8, 33, 16388, 0, "all", 4), (8, 33, 16386, 0, "all", 2),
    (2, 17, 24580, 8, "all", 4), (11, 29, 4092, 0, "all", 4), (16, 7, 6146, 4, "all", 2),
    (1, 1000, 2044, 0, "all", 4), (1, 3, 1, 0, "all", 1),
]


# Both residual_out store policies (streaming and write-back stores) on the row and the
# scalar kernels: the same bits either way, in one span and in several.
@pytest.mark.parametrize("W,T,H,variant", [(4, 130, 2048, ROW), (2, 33, 1000, ROW), (4, 130, 2047, SCALAR),
                                           (3, 9, 8193, SCALAR), (12, 17, 4096, ROW), (9, 5, 1001, SCALAR)])
@pytest.mark.parametrize("store", [1, 2])
def test_residual_out_store_policies(W, T, H, variant, store):
    plan, _ = parity(W, T, H, variant=variant, tuning=dict(residual_out_store=store), seed=T + H + store)
    assert plan["residual_out_cached"] == store - 1


# More than 8 ranks with enough rows, or 6-8 ranks on power-of-two workgroups: the automatic
# plan is the scalar kernel's rank loop.
@pytest.mark.parametrize("W,T,H", [(12, 1024, 4096), (16, 2048, 2048), (9, 1030, 1000), (11, 1024, 2046),
                                   (12, 1024, 8192), (10, 1100, 6000), (8, 2048, 2048), (6, 2100, 4096),
                                   (7, 2048, 8184), (8, 2048, 4095), (8, 2049, 5119), (8, 2048, 8190)])
def test_many_ranks_scalar_plan(W, T, H):
    plan, _ = parity(W, T, H, seed=W * 1000 + H)
    assert plan["variant"] == SCALAR


# Rows whose stride is not a multiple of 128 bytes, with enough rows: the automatic plan
# is the scalar kernel, 8-byte loads, lanes rotated onto whole lines row by row.
@pytest.mark.parametrize("W,T,H", [(4, 4096, 2040), (1, 16384, 1000), (2, 4096, 6000), (8, 4096, 3000),
                                   (5, 4100, 8136), (3, 4097, 1544)])
def test_line_offset_rows_scalar_plan(W, T, H):
    plan, _ = parity(W, T, H, seed=W * 1000 + H + 7)
    assert plan["variant"] == SCALAR and plan["elems_per_load"] == 4 and plan["rank_loop"] == 0


# Kernels with preloaded arguments (the flat-argument twins) and kernels taking one
# argument block: the same bits, each forced on row kernels of several lane layouts and
# scalar kernels of every load width (specialised W <= 8), small and large calls.
@pytest.mark.parametrize("W,T,H,variant", [(1, 300, 2048, ROW), (2, 1000, 1024, ROW), (3, 37, 8192, ROW),
                                           (4, 4096, 2048, ROW), (5, 64, 5120, ROW), (6, 33, 2048, ROW),
                                           (7, 100, 4096, ROW), (8, 129, 16384, ROW), (4, 130, 2047, SCALAR),
                                           (3, 77, 2046, SCALAR), (8, 200, 2044, SCALAR), (1, 65, 8193, SCALAR),
                                           (4, 4096, 2040, AUTO)])
@pytest.mark.parametrize("preload", [1, 2])
def test_kernarg_preload_paths(W, T, H, variant, preload):
    plan, _ = parity(W, T, H, variant=variant, tuning=dict(kernarg_preload=preload), seed=W + T + H + preload)
    assert plan["kernarg_preload"] == (preload == 2), plan


def _shifted(t, off, dev):
    """A copy of CPU tensor t on the GPU, starting `off` bytes past a 256-byte boundary."""
    buf = torch.zeros(t.numel() + 16, dtype=torch.bfloat16, device=dev)
    view = buf[off // 2:off // 2 + t.numel()].view(t.shape)
    view.copy_(t.to(dev))
    return view


@pytest.mark.parametrize("W,T,H,off,which,elems", SCALAR_WIDTHS)
def test_scalar_load_widths(W, T, H, off, which, elems):
    where = "scalar width W=%d T=%d H=%d offset=%d on %s" % (W, T, H, off, which)
    say("case " + where)
    dev = torch.device("cuda", 0)
    x, res, w = inputs(W, T, H, seed=H + off + W)
    o_all = off if which == "all" else 0
    xs = [_shifted(x[r], off if (which in ("all", "partial") and r == W - 1) or which == "all" else 0, dev)
          for r in range(W)]
    rs = _shifted(res, off if which in ("all", "residual") else 0, dev)
    ws = _shifted(w, off if which in ("all", "weight") else 0, dev)
    ro = _shifted(torch.zeros(T, H, dtype=torch.bfloat16), o_all, dev)
    no = _shifted(torch.zeros(T, H, dtype=torch.bfloat16), off if which in ("all", "norm_out") else 0, dev)
    o = op()
    plan = o.plan(xs, rs, ws, 1e-6, ro, no)
    assert plan["variant"] == SCALAR and plan["elems_per_load"] == elems, plan
    o(xs, rs, ws, 1e-6, ro, no)
    torch.cuda.synchronize()
    n = assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, res, w, 1e-6), where)
    say("  plan %s, norm_out not bit-identical: %d of %d" % (plan, n, no.numel()))


@pytest.mark.parametrize("elems", [1, 2, 4])
@pytest.mark.parametrize("T,H", [(4096, 2048), (3, 16392), (5, 1000)])
def test_scalar_tuned_narrower_loads(elems, T, H):
    """Tuning caps the load width: the same rows through 2-, 4- and 8-byte loads."""
    plan, _ = parity(4, T, H, variant=SCALAR, tuning=dict(scalar_elems=elems), seed=T + elems)
    assert plan["elems_per_load"] == min(elems, 4 if H % 4 == 0 else (2 if H % 2 == 0 else 1))


# The largest hidden size (ARRMS_MAX_HIDDEN) and the largest world size together,
# on the vector variants the planner can pick for them.
@pytest.mark.parametrize("W,T,H,variant", [(16, 3, 65536, AUTO), (8, 5, 65536, SPLITH), (16, 2, 65528, SPLITH),
                                           (8, 4, 16384, ROW), (16, 9, 4096, ROW)])
def test_largest_sizes(W, T, H, variant):
    plan, _ = parity(W, T, H, variant=variant, seed=H + W)
    if variant != AUTO:
        assert plan["variant"] == variant


# One or two ranks with short rows take four vectors per lane in sub-wave row groups
# when the automatic plan finds enough rows (ragged T, a non-power-of-two row).
@pytest.mark.parametrize("W,T,H", [(1, 4096, 2048), (1, 8192, 1024), (1, 16384, 512), (1, 4097, 1536),
                                   (1, 2049, 2048), (2, 8191, 1024), (2, 4096, 2048), (2, 8192, 512),
                                   (2, 2047, 1536)])
def test_few_ranks_short_rows(W, T, H):
    plan, _ = parity(W, T, H, seed=T + H + W)
    assert plan["variant"] == ROW and plan["vec_per_thread"] == 4 and plan["threads_per_row"] <= 64


def _row_tunings(W, H):
    nvec = H // 8
    out = []
    for vpt in (1, 2, 4, 8):
        we = W if (W <= 8 or W == 16) else 16
        if (we + 2) * vpt > 40:
            continue
        for tpr in (16, 32, 64, 128, 192, 256, 320, 512, 640, 1024):
            cap = (512 if vpt == 1 else 256) if we > 8 else (1024 if vpt == 1 else (512 if vpt <= 4 else 256))
            if tpr * vpt >= nvec and tpr <= cap and tpr * vpt < 2 * nvec + 64:
                out.append(dict(vec_per_thread=vpt, threads_per_row=tpr))
    return out


ROW_TUNING_CASES = [(W, H, t) for W, H in [(4, 2048), (8, 8192), (8, 5120), (2, 128), (3, 1000)]
                    for t in _row_tunings(W, H)]


@pytest.mark.parametrize("W,H,tuning", ROW_TUNING_CASES,
                         ids=["W%d-H%d-v%d-t%d" % (W, H, t["vec_per_thread"], t["threads_per_row"])
                              for W, H, t in ROW_TUNING_CASES])
def test_row_tuning_grid(W, H, tuning):
    """Every row-kernel instance and lane-group size the planner can pick or the benchmark
    sweeps, on a ragged row count."""
    plan, _ = parity(W, 67, H, variant=ROW, tuning=tuning, seed=7)
    assert plan["vec_per_thread"] == tuning["vec_per_thread"]
    assert plan["threads_per_row"] == tuning["threads_per_row"]


SPLITH_CASES = [(W, H, b, v) for W, H in [(4, 2048), (8, 8192), (8, 5120), (16, 2048)]
                for b in (64, 128, 256, 512, 1024) for v in (1, 2)
                if not (W > 8 and (v > 1 or b > 512))]


@pytest.mark.parametrize("W,H,block,vpt", SPLITH_CASES)
def test_splith_tuning_grid(W, H, block, vpt):
    plan, _ = parity(W, 5, H, variant=SPLITH, tuning=dict(vec_per_thread=vpt, splith_block=block), seed=9)
    assert plan["block"] == block and plan["vec_per_thread"] == vpt


XCD_CASES = [(W, T, H, variant, xcd) for W, T, H in [(4, 4096, 2048), (8, 77, 5120), (4, 3, 2048)]
             for variant in (ROW, SPLITH) for xcd in (0, 1, 7, 64, 10 ** 6)]


@pytest.mark.parametrize("W,T,H,variant,xcd", XCD_CASES)
def test_xcd_mapping(W, T, H, variant, xcd):
    """The XCD block mapping (with its padding workgroups) changes no result bit."""
    plan, _ = parity(W, T, H, variant=variant, tuning=dict(xcd_chunk=xcd), seed=21 + T)
    k = plan["xcd_chunk"]
    assert k == min(xcd, -(-plan["blocks"] // 8))
    if k:
        assert plan["grid"] % (8 * k) == 0 and 0 <= plan["grid"] - plan["blocks"] < 8 * k


# ------------------------------------------------------------ semantics and edge cases
def test_partials_as_a_token_slice_of_a_larger_buffer():
    """[W, T, H] partials that are a token slice of a [W, T2, H] buffer (not contiguous as a
    whole, each rank's rows contiguous) go through the per-rank pointer path."""
    say("case partials token slice")
    W, T, H = 4, 50, 2048
    x, res, w = inputs(W, T, H, seed=21)
    big = torch.zeros((W, T + 30, H), dtype=torch.bfloat16, device="cuda")
    big[:, 10:10 + T].copy_(x.to("cuda"))
    xs = big[:, 10:10 + T]
    assert not xs.is_contiguous()
    ro, no = op()(xs, res.to("cuda"), w.to("cuda"), 1e-6)
    torch.cuda.synchronize()
    assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, res, w, 1e-6), "token slice")


@pytest.mark.parametrize("variant", [ROW, SPLITH, SCALAR])
def test_in_place_residual(variant):
    parity(4, 130, 2048, variant=variant, inplace=True, seed=3)


def test_misaligned_pointers_take_scalar_path():
    say("case misaligned +2 bytes, W=3 T=21 H=2048")
    W, T, H = 3, 21, 2048
    x, res, w = inputs(W, T, H, seed=5)
    dev = torch.device("cuda", 0)
    n = T * H

    def shifted(t):
        buf = torch.zeros(t.numel() + 8, dtype=torch.bfloat16, device=dev)
        view = buf[1:1 + t.numel()].view(t.shape)
        view.copy_(t.to(dev))
        return view

    xs = [shifted(x[r]) for r in range(W)]
    rs, ws = shifted(res), shifted(w)
    ro = torch.zeros(n + 8, dtype=torch.bfloat16, device=dev)[1:1 + n].view(T, H)
    no = torch.zeros(n + 8, dtype=torch.bfloat16, device=dev)[1:1 + n].view(T, H)
    o = op()
    assert o.plan(xs, rs, ws, 1e-6, ro, no)["variant"] == SCALAR
    o(xs, rs, ws, 1e-6, ro, no)
    torch.cuda.synchronize()
    assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, res, w, 1e-6), "misaligned")


@pytest.mark.parametrize("variant", [ROW, SPLITH, SCALAR])
def test_guard_bands_untouched(variant):
    """Outputs sit between canary bands; no kernel writes outside its outputs."""
    say("case guard bands variant=%s" % VNAME[variant])
    W, T, H, G = 4, 77, 2048, 4096
    x, res, w = inputs(W, T, H, seed=12)
    dev = torch.device("cuda", 0)
    canary = torch.full((2 * G + T * H,), 0x5A5A, dtype=torch.int16, device=dev)
    ro_buf, no_buf = canary.clone(), canary.clone()
    ro = ro_buf.view(torch.bfloat16)[G:G + T * H].view(T, H)
    no = no_buf.view(torch.bfloat16)[G:G + T * H].view(T, H)
    o = op()
    o.set_variant(variant)
    try:
        o(x.to(dev), res.to(dev), w.to(dev), 1e-6, ro, no)
        torch.cuda.synchronize()
    finally:
        o.set_variant(AUTO)
    for buf in (ro_buf, no_buf):
        b = buf.cpu()
        assert bool((b[:G] == 0x5A5A).all()) and bool((b[G + T * H:] == 0x5A5A).all())
    assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, res, w, 1e-6), "guard")


@pytest.mark.parametrize("variant", [AUTO, ROW, SPLITH, SCALAR])
@pytest.mark.parametrize("T", [1, 16, 128])
def test_deterministic(variant, T):
    say("case determinism variant=%s T=%d" % (VNAME[variant], T))
    x, res, w = inputs(4, T, 2048, seed=13)
    first = run(x, res, w, 1e-6, variant=variant)
    for _ in range(3):
        again = run(x, res, w, 1e-6, variant=variant)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def test_splith_back_to_back_calls_share_workspace():
    """Many split-H calls in a row on one handle and stream, each on different data and
    row counts, all through the handle's one workspace."""
    say("case split-H back-to-back")
    dev = torch.device("cuda", 0)
    o = op()
    cases = [inputs(4, T, 2048, seed=200 + T) for T in (1, 5, 16, 40, 128, 3)]
    dev_in = [(x.to(dev), r.to(dev), w.to(dev)) for x, r, w in cases]
    o.set_variant(SPLITH)
    try:
        outs = []
        for rep in range(20):
            for xd, rd, wd in dev_in:
                outs.append(o(xd, rd, wd, 1e-6))
        torch.cuda.synchronize()
    finally:
        o.set_variant(AUTO)
    for i, (ro, no) in enumerate(outs[-len(cases):]):
        x, r, w = cases[i]
        assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, r, w, 1e-6), "b2b %d" % i)
    for i, (ro, no) in enumerate(outs[:len(cases)]):
        x, r, w = cases[i]
        assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, r, w, 1e-6), "b2b first %d" % i)


def test_zero_tokens_enqueues_nothing():
    say("case T=0")
    dev = torch.device("cuda", 0)
    e = torch.empty((0, 2048), dtype=torch.bfloat16, device=dev)
    w = torch.ones(2048, dtype=torch.bfloat16, device=dev)
    rc = A.arrms_fused(op().handle, [e.data_ptr()] * 4, 4, 0, 2048, e.data_ptr(), w.data_ptr(), 1e-6,
                       e.data_ptr(), e.data_ptr(), 0)
    assert rc == A.ARRMS_OK


@pytest.mark.parametrize("variant", [ROW, SPLITH, SCALAR])
def test_zero_row_with_zero_eps_gives_nan_like_oracle(variant):
    say("case zero rows eps=0 variant=%s" % VNAME[variant])
    x, res, w = inputs(2, 9, 2048, seed=14)
    x[:, 3] = 0
    res[3] = 0
    ro, no, _ = run(x, res, w, 0.0, variant=variant)
    ref = reference(x, res, w, 0.0)
    assert np.isnan(bf16_values(no[3])).all()
    assert_parity(ro, no, ref, "zero-row eps=0")


@pytest.mark.parametrize("variant", [ROW, SPLITH, SCALAR])
def test_zero_residual_exposes_reduced(variant):
    """With residual = 0, residual_out equals the BF16 rank sum `reduced` (by value)."""
    say("case reduced via zero residual variant=%s" % VNAME[variant])
    x, res, w = inputs(8, 50, 5120, seed=15, outlier_p=0.01)
    res.zero_()
    ro, no, _ = run(x, res, w, 1e-6, variant=variant)
    ref = reference(x, res, w, 1e-6)
    np.testing.assert_array_equal(bf16_values(ro), bf16_values(ref["reduced"]))
    assert_parity(ro, no, ref, "zero residual")


def test_non_default_stream():
    say("case non-default stream")
    s = torch.cuda.Stream(device=0)
    x, res, w = inputs(4, 300, 2048, seed=16)
    with torch.cuda.stream(s):
        ro, no, _ = run(x, res, w, 1e-6, stream=s)
    assert_parity(ro, no, reference(x, res, w, 1e-6), "stream")


def test_errors_on_a_device_handle():
    say("case error returns")
    dev = torch.device("cuda", 0)
    rc, h = A.arrms_create(0, 4, 8, 2048)
    assert rc == A.ARRMS_OK
    try:
        t = torch.zeros((16, 4096), dtype=torch.bfloat16, device=dev)
        w = torch.ones(4096, dtype=torch.bfloat16, device=dev)
        p = t.data_ptr()
        big = torch.zeros((3, 16, 4096), dtype=torch.bfloat16, device=dev)
        q = [big[i].data_ptr() for i in range(3)]
        ok = lambda W, T, H: (h, [p] * W, W, T, H, p, w.data_ptr(), 1e-6, q[1], q[2], 0)
        assert A.arrms_fused(*ok(4, 8, 2048)) == A.ARRMS_OK
        assert A.arrms_fused(*ok(5, 8, 2048)) == A.ARRMS_ERR_INVALID_ARG    # world > max_world
        assert A.arrms_fused(*ok(4, 9, 2048)) == A.ARRMS_ERR_INVALID_ARG    # tokens > max_tokens
        assert A.arrms_fused(*ok(4, 8, 4096)) == A.ARRMS_ERR_INVALID_ARG    # hidden > max_hidden
        bad_eps = list(ok(4, 8, 2048))
        bad_eps[7] = -1.0
        assert A.arrms_fused(*bad_eps) == A.ARRMS_ERR_INVALID_ARG
        torch.cuda.synchronize()
        assert A.arrms_last_hip_error(h) == 0
    finally:
        assert A.arrms_destroy(h) == A.ARRMS_OK


def test_create_destroy_cycles():
    say("case create/destroy cycles")
    for i in range(5):
        rc, h = A.arrms_create(0, 8, 1000 + i, 8192)
        assert rc == A.ARRMS_OK and h
        assert A.arrms_destroy(h) == A.ARRMS_OK
    rc, h = A.arrms_create(0, 4, 2 ** 31 - 1, 65536)  # workspace far beyond device memory
    assert rc == A.ARRMS_ERR_OOM and h is None
    # the failed allocation leaves no stale error behind for the next launch check
    torch.zeros(1000, device="cuda").add_(1)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,variant", [("row", ROW), ("splith", SPLITH), ("scalar", SCALAR)])
def test_force_variant_environment(name, variant, monkeypatch):
    """ARRMS_FORCE_VARIANT is read once, when a handle is created."""
    say("case ARRMS_FORCE_VARIANT=%s" % name)
    monkeypatch.setenv("ARRMS_FORCE_VARIANT", name)
    o = A.FusedReduceResidualRMSNorm(4, 64, 2048, device=0)
    monkeypatch.delenv("ARRMS_FORCE_VARIANT")
    try:
        x, res, w = inputs(4, 40, 2048, seed=500)
        dev = torch.device("cuda", 0)
        xd, rd, wd = x.to(dev), res.to(dev), w.to(dev)
        assert o.plan(xd, rd, wd, 1e-6)["variant"] == variant
        ro, no = o(xd, rd, wd, 1e-6)
        torch.cuda.synchronize()
        assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, res, w, 1e-6), "env " + name)
    finally:
        o.close()


def test_bound_call_matches_plain_call():
    say("case bound call")
    dev = torch.device("cuda", 0)
    x, res, w = inputs(4, 77, 2048, seed=600)
    xd, rd, wd = x.to(dev), res.to(dev), w.to(dev)
    o = op()
    call = o.bind(xd, rd, wd, 1e-6)
    ro, no = call()
    call()  # idempotent: same inputs, same outputs
    torch.cuda.synchronize()
    assert_parity(synth.bits(ro.cpu()), synth.bits(no.cpu()), reference(x, res, w, 1e-6), "bound call")
    with pytest.raises(A.ArrmsError):
        o.bind(xd, rd, wd, -1.0)
