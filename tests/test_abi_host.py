"""The C-ABI library on the host: it loads, exports every declared symbol, and its
host-only validation and variant planning (arrms_plan) behave as include/arrms.h says.
No kernel is launched and no device memory is touched: pointers are fake integers
that the planner compares but never dereferences."""
import os
import re

import pytest

import residual_add_rmsnorm_arrms_amd as A

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "arrms.h")
CU = 256
LIM = dict(max_world=16, max_tokens=20000, max_hidden=65536)
BASE = 0x7F0000000000


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(A.LIB_PATH):
        from residual_add_rmsnorm_arrms_amd import build
        build.build()
    return A.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(arrms_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    assert sorted(A.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def declaration_comment(name):
    """The comment block directly above the declaration of `name` in the header."""
    text = open(HEADER).read()
    m = re.search(r"(/\*(?:(?!\*/).)*\*/)\s*(?:int|const char\*)\s+%s\s*\(" % name, text, re.S)
    assert m, name
    return m.group(1)


@pytest.mark.parametrize("name", ["arrms_create", "arrms_fused", "arrms_destroy", "arrms_status_string",
                                  "arrms_reduce"])
def test_boundary_exports_cite_a_section_of_the_page(name):
    """Each entry point of the boundary names the passage of the page that defines it."""
    c = declaration_comment(name)
    assert re.search(r"section (Summary|Implementation \d)", c), name
    # the comment belongs to this declaration only (no other declaration in between)
    assert not re.search(r"^\s*(int|const char\*)\s+arrms_\w+\s*\(", c, re.M)


def test_status_strings():
    assert A.arrms_status_string(A.ARRMS_OK) == "ok"
    assert A.arrms_status_string(A.ARRMS_ERR_INVALID_ARG) == "invalid argument"
    assert A.arrms_status_string(A.ARRMS_ERR_UNSUPPORTED) == "unsupported shape or variant"
    assert A.arrms_status_string(A.ARRMS_ERR_HIP) == "HIP runtime error"
    assert A.arrms_status_string(A.ARRMS_ERR_OOM) == "out of device memory"
    assert "static scratch" in A.arrms_status_string(A.ARRMS_ERR_SCRATCH)
    assert A.arrms_status_string(99) == "unknown status"


def bufs(W, T, H, align=256, off=0):
    """Disjoint fake buffers: W partials, residual, weight, residual_out, norm_out."""
    n = T * H * 2
    step = (n + 2 * H + 4096 + align - 1) // align * align
    ptrs = [BASE + i * step + off for i in range(W + 4)]
    return dict(partials=ptrs[:W], residual=ptrs[W], weight=ptrs[W + 1], residual_out=ptrs[W + 2],
                norm_out=ptrs[W + 3])


def grid_of(p):
    k = p["xcd_chunk"]
    return -(-p["blocks"] // (8 * k)) * (8 * k) if k else p["blocks"]


def plan(W, T, H, variant=A.ARRMS_VARIANT_AUTO, tuning=None, eps=1e-6, cu=CU, lim=LIM, **over):
    b = bufs(W, T, H)
    b.update(over)
    return A.arrms_plan(cu, variant, tuning, lim["max_world"], lim["max_tokens"], lim["max_hidden"],
                        b["partials"], W, T, H, b["residual"], b["weight"], eps, b["residual_out"], b["norm_out"])


def test_prefill_shape_uses_row_variant():
    rc, p = plan(4, 4096, 2048)
    assert rc == A.ARRMS_OK
    assert p["variant"] == A.ARRMS_VARIANT_ROW
    assert p["threads_per_row"] * p["vec_per_thread"] >= 2048 // 8
    assert p["blocks"] * p["rows_per_block"] >= 4096
    assert p["block"] % 64 == 0 and p["block"] <= 1024
    assert p["kernels"] == 1 and p["grid"] == grid_of(p)


@pytest.mark.parametrize("W,T,H", [(8, 8192, 8192), (8, 16383, 5120), (2, 4, 128), (4, 1000, 64), (1, 5, 8),
                                   (16, 300, 2048), (11, 300, 4096), (3, 77, 16384)])
def test_row_plans_cover_the_row(W, T, H):
    rc, p = plan(W, T, H, variant=A.ARRMS_VARIANT_ROW)
    assert rc == A.ARRMS_OK, (W, T, H)
    nvec = H // 8
    assert p["threads_per_row"] * p["vec_per_thread"] >= nvec
    assert p["blocks"] * p["rows_per_block"] >= T > (p["blocks"] - 1) * p["rows_per_block"]
    assert p["grid"] == grid_of(p)
    assert p["block"] == p["threads_per_row"] * p["rows_per_block"] and p["block"] % 64 == 0
    assert p["threads_per_row"] in (16, 32) or p["threads_per_row"] % 64 == 0
    we = W if (W <= 8 or W == 16) else 16
    assert (we + 2) * p["vec_per_thread"] <= 40


@pytest.mark.parametrize("W,T,H", [(4, 1, 2048), (4, 16, 2048), (8, 1, 8192), (8, 3, 65536), (16, 2, 2048),
                                   (4, 5000, 32768), (12, 1, 24576)])
def test_splith_plans(W, T, H):
    rc, p = plan(W, T, H, variant=A.ARRMS_VARIANT_SPLITH)
    assert rc == A.ARRMS_OK, (W, T, H)
    chunk = p["block"] * p["vec_per_thread"]
    assert p["chunks_per_row"] == -(-(H // 8) // chunk)
    assert p["chunks_per_row"] <= -(-(65536 // 8) // 64)
    assert p["blocks"] == T * p["chunks_per_row"] and p["kernels"] == 2
    assert p["grid"] == grid_of(p)
    assert p["block"] % 64 == 0 and p["block"] <= (512 if W > 8 else 1024)


def test_auto_selection():
    assert plan(4, 1, 2048)[1]["variant"] == A.ARRMS_VARIANT_ROW         # decode: one kernel is faster
    assert plan(4, 4096, 2048)[1]["variant"] == A.ARRMS_VARIANT_ROW      # prefill
    assert plan(4, 4096, 32768)[1]["variant"] == A.ARRMS_VARIANT_SPLITH  # H beyond the row kernels
    assert plan(4, 100, 1000)[1]["variant"] == A.ARRMS_VARIANT_ROW       # H % 8 == 0
    assert plan(4, 100, 1001)[1]["variant"] == A.ARRMS_VARIANT_SCALAR    # H % 8 != 0
    b = bufs(4, 100, 2048)
    rc, p = plan(4, 100, 2048, residual=b["residual"] + 2)               # 2-byte aligned only
    assert rc == A.ARRMS_OK and p["variant"] == A.ARRMS_VARIANT_SCALAR
    t = A.arrms_tuning_t.make(splith_max_tokens=8)
    assert plan(4, 8, 2048, tuning=t)[1]["variant"] == A.ARRMS_VARIANT_SPLITH  # crossover moved up
    assert plan(4, 9, 2048, tuning=t)[1]["variant"] == A.ARRMS_VARIANT_ROW


def test_xcd_mapping_plans():
    rc, p = plan(4, 4096, 2048, tuning=A.arrms_tuning_t.make(xcd_chunk=0))
    assert rc == A.ARRMS_OK and p["xcd_chunk"] == 0 and p["grid"] == p["blocks"]
    rc, p = plan(4, 3, 2048, tuning=A.arrms_tuning_t.make(xcd_chunk=1))
    assert p["xcd_chunk"] == 1 and p["grid"] == 8 and p["blocks"] == 3
    rc, p = plan(4, 1000, 2048, tuning=A.arrms_tuning_t.make(xcd_chunk=16))
    assert p["xcd_chunk"] == 16 and p["grid"] == 1024 and p["blocks"] == 1000
    rc, p = plan(4, 1000, 2048, tuning=A.arrms_tuning_t.make(xcd_chunk=10 ** 6))  # clamped to blocks / 8
    assert p["xcd_chunk"] == 125 and p["grid"] == 1000
    rc, p = plan(4, 3, 2048)
    assert p["xcd_chunk"] == 0 and p["grid"] == 3                       # small grids: no padding
    rc, p = plan(4, 100, 1001)                                          # scalar: XCD runs like the row kernel
    assert p["variant"] == A.ARRMS_VARIANT_SCALAR and p["xcd_chunk"] == 13 and p["grid"] == 104
    rc, p = plan(4, 63, 1001)
    assert p["variant"] == A.ARRMS_VARIANT_SCALAR and p["xcd_chunk"] == 0 and p["grid"] == 63


@pytest.mark.parametrize("blocks,k", [(8, 1), (13, 1), (100, 3), (64, 8), (1000, 16), (4096, 512), (77, 10)])
def test_xcd_mapping_is_a_bijection(blocks, k):
    """The kernels' logical-block formula, run on the host over the planned grid: every
    logical block exactly once, padding workgroups only past the end."""
    grid = -(-blocks // (8 * k)) * (8 * k)
    seen = []
    for b in range(grid):
        x, i = b % 8, b // 8
        j = i // k
        l = (j * 8 + x) * k + (i - j * k)
        if l < blocks:
            seen.append(l)
    assert sorted(seen) == list(range(blocks))


def test_forced_variant_unsupported():
    assert plan(4, 10, 1000 + 1, variant=A.ARRMS_VARIANT_ROW)[0] == A.ARRMS_ERR_UNSUPPORTED
    assert plan(4, 10, 1001, variant=A.ARRMS_VARIANT_SPLITH)[0] == A.ARRMS_ERR_UNSUPPORTED
    assert plan(4, 10, 32768, variant=A.ARRMS_VARIANT_ROW)[0] == A.ARRMS_ERR_UNSUPPORTED
    assert plan(4, 10, 1001, variant=A.ARRMS_VARIANT_SCALAR)[0] == A.ARRMS_OK
    t = A.arrms_tuning_t.make(vec_per_thread=8)
    assert plan(8, 10, 2048, variant=A.ARRMS_VARIANT_ROW, tuning=t)[0] == A.ARRMS_ERR_UNSUPPORTED  # registers


@pytest.mark.parametrize("T,H", [(2 ** 24, 8), (2 ** 24 - 3, 64), (2 ** 22 + 1, 2048), (2 ** 31 - 1, 8),
                                 (2 ** 31 - 1, 2048)])
def test_huge_token_counts(T, H):
    """Block counts are computed without int overflow; a plan whose grid would exceed
    2^32 work-items (the launch limit) is refused as unsupported, never truncated."""
    lim = dict(max_world=8, max_tokens=2 ** 31 - 1, max_hidden=65536)
    for variant in (A.ARRMS_VARIANT_AUTO, A.ARRMS_VARIANT_ROW, A.ARRMS_VARIANT_SCALAR):
        rc, p = plan(4, T, H, variant=variant, lim=lim)
        assert rc in (A.ARRMS_OK, A.ARRMS_ERR_UNSUPPORTED), (variant, rc)
        if rc == A.ARRMS_ERR_UNSUPPORTED:
            assert T * min(H, 64) > 2 ** 32 // 256, (T, H, variant)   # only refused when genuinely too big
            continue
        assert p["grid"] * p["block"] <= 2 ** 32 - 1
        assert p["blocks"] > 0 and p["blocks"] * p["rows_per_block"] >= T
        assert (p["blocks"] - 1) * p["rows_per_block"] < T
    rc, p = A.arrms_plan_reduce(CU, None, 8, 2 ** 31 - 1, 65536, [BASE + i * 2 ** 44 for i in range(4)], 4, T, H,
                                BASE + 5 * 2 ** 44)
    assert rc in (A.ARRMS_OK, A.ARRMS_ERR_UNSUPPORTED)
    if rc == A.ARRMS_OK:
        assert p["grid"] * p["block"] <= 2 ** 32 - 1 and p["blocks"] * 256 * 8 * p["vec_per_thread"] >= T * H


def test_tokens_zero_is_ok_and_plans_nothing():
    rc, p = A.arrms_plan(CU, 0, None, 4, 10, 2048, None, 4, 0, 2048, 0, 0, 1e-6, 0, 0)
    assert rc == A.ARRMS_OK and p["grid"] == 0


@pytest.mark.parametrize("case", [
    dict(W=0), dict(W=17), dict(T=-1), dict(T=20001), dict(H=0), dict(H=65537),
    dict(eps=-1e-6), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(cu=0), dict(variant=4), dict(variant=-1),
])
def test_invalid_sizes(case):
    W, T, H = case.get("W", 4), case.get("T", 16), case.get("H", 2048)
    b = bufs(max(W, 1), max(T, 1), max(H, 1))
    parts = (b["partials"] * 17)[:max(W, 1)]
    rc, p = A.arrms_plan(case.get("cu", CU), case.get("variant", 0), None, 16, 20000, 65536, parts, W, T, H,
                         b["residual"], b["weight"], case.get("eps", 1e-6), b["residual_out"], b["norm_out"])
    assert rc == A.ARRMS_ERR_INVALID_ARG and p["grid"] == 0


def test_world_above_handle_limit():
    lim = dict(LIM, max_world=4)
    assert plan(5, 16, 2048, lim=lim)[0] == A.ARRMS_ERR_INVALID_ARG
    assert plan(4, 16, 2048, lim=lim)[0] == A.ARRMS_OK


@pytest.mark.parametrize("field", ["residual", "weight", "residual_out", "norm_out"])
def test_null_pointers(field):
    assert plan(4, 16, 2048, **{field: 0})[0] == A.ARRMS_ERR_INVALID_ARG


def test_null_partial_and_odd_alignment():
    b = bufs(4, 16, 2048)
    assert plan(4, 16, 2048, partials=[b["partials"][0], 0, *b["partials"][2:]])[0] == A.ARRMS_ERR_INVALID_ARG
    assert plan(4, 16, 2048, norm_out=b["norm_out"] + 1)[0] == A.ARRMS_ERR_INVALID_ARG
    assert plan(4, 16, 2048, partials=[b["partials"][0] + 1, *b["partials"][1:]])[0] == A.ARRMS_ERR_INVALID_ARG


def test_aliasing_rules():
    b = bufs(4, 16, 2048)
    n = 16 * 2048 * 2
    assert plan(4, 16, 2048, residual_out=b["residual"])[0] == A.ARRMS_OK                # in place
    assert plan(4, 16, 2048, residual_out=b["residual"] + 64)[0] == A.ARRMS_ERR_INVALID_ARG  # partial overlap
    assert plan(4, 16, 2048, norm_out=b["residual_out"] + n - 2)[0] == A.ARRMS_ERR_INVALID_ARG
    assert plan(4, 16, 2048, norm_out=b["residual_out"] + n)[0] == A.ARRMS_OK              # adjacent is fine
    assert plan(4, 16, 2048, norm_out=b["residual"])[0] == A.ARRMS_ERR_INVALID_ARG
    assert plan(4, 16, 2048, residual_out=b["partials"][2])[0] == A.ARRMS_ERR_INVALID_ARG
    assert plan(4, 16, 2048, norm_out=b["weight"] - 2)[0] == A.ARRMS_ERR_INVALID_ARG
    # inputs may overlap each other (read-only)
    p = b["partials"]
    assert plan(4, 16, 2048, partials=[p[0], p[0], p[0], p[0]])[0] == A.ARRMS_OK


@pytest.mark.parametrize("t", [(3, 0, 0, -1, -1, 0), (0, 48, 0, -1, -1, 0), (0, 2048, 0, -1, -1, 0),
                               (0, 0, 100, -1, -1, 0), (0, 0, 0, -2, -1, 0), (0, 0, 0, -1, -2, 0),
                               (0, 0, 0, -1, -1, 3), (0, 0, 0, -1, -1, -1), (0, 0, 0, -1, -1, 128)])
def test_invalid_tuning(t):
    assert plan(4, 16, 2048, tuning=A.arrms_tuning_t(*t))[0] == A.ARRMS_ERR_INVALID_ARG


def test_null_handle_calls():
    assert A.arrms_destroy(None) == A.ARRMS_OK
    assert A.arrms_last_hip_error(None) == -1
    assert A.arrms_set_variant(None, 0) == A.ARRMS_ERR_INVALID_ARG
    assert A.arrms_set_tuning(None, None) == A.ARRMS_ERR_INVALID_ARG
    b = bufs(4, 16, 2048)
    rc, p = A.arrms_query_plan(None, b["partials"], 4, 16, 2048, b["residual"], b["weight"], 1e-6,
                               b["residual_out"], b["norm_out"])
    assert rc == A.ARRMS_ERR_INVALID_ARG
    assert A.arrms_fused(None, b["partials"], 4, 16, 2048, b["residual"], b["weight"], 1e-6, b["residual_out"],
                         b["norm_out"], 0) == A.ARRMS_ERR_INVALID_ARG


def test_create_rejects_bad_limits():
    for args in [(0, 0, 16, 2048), (0, 17, 16, 2048), (0, 4, -1, 2048), (0, 4, 16, 0), (0, 4, 16, 65537),
                 (-1, 4, 16, 2048)]:
        rc, h = A.arrms_create(*args)
        assert rc == A.ARRMS_ERR_INVALID_ARG and h is None


@pytest.mark.parametrize("W,T,H,variant,vpt,tpr,k", [
    (4, 4096, 2048, A.ARRMS_VARIANT_ROW, 1, 256, 64),      # prefill: 256-lane rows, 64-row XCD runs
    (8, 8192, 8192, A.ARRMS_VARIANT_SCALAR, 0, 1024, 16),  # large_hidden: the rank loop on 1024 lanes
    (8, 16383, 5120, A.ARRMS_VARIANT_ROW, 2, 512, 16),     # 8-wave rows beat exact 5-wave rows
    (4, 16, 2048, A.ARRMS_VARIANT_ROW, 1, 256, 0),         # decode, small rows: one kernel
    (8, 1, 8192, A.ARRMS_VARIANT_SPLITH, 1, 64, 0),        # decode, large rows: split over CUs
    (8, 128, 8192, A.ARRMS_VARIANT_ROW, 2, 512, 16),
    (1, 4096, 2048, A.ARRMS_VARIANT_ROW, 4, 64, 32),       # one rank, short rows: 4 vectors per lane
    (1, 8192, 1024, A.ARRMS_VARIANT_ROW, 4, 32, 32),
    (1, 16384, 512, A.ARRMS_VARIANT_ROW, 4, 16, 32),
    (1, 4096, 512, A.ARRMS_VARIANT_ROW, 1, 64, 128),       # ... unless fewer than 2 workgroups per CU
    (1, 1024, 2048, A.ARRMS_VARIANT_ROW, 1, 256, 128),
    (2, 8192, 1024, A.ARRMS_VARIANT_ROW, 4, 32, 32),       # two ranks: four vectors while one round fits
    (2, 16384, 1024, A.ARRMS_VARIANT_ROW, 1, 128, 128),    # ... not beyond four workgroups per CU
    (2, 4096, 2048, A.ARRMS_VARIANT_ROW, 4, 64, 32),
    (3, 2048, 1536, A.ARRMS_VARIANT_ROW, 1, 256, 128),     # three ranks keep one vector per lane
    (4, 4096, 2048, A.ARRMS_VARIANT_ROW, 1, 256, 64),      # four ranks keep one vector per lane
])
def test_measured_automatic_choices(W, T, H, variant, vpt, tpr, k):
    """The automatic choices the MI355X measurements led to (speed only; results are
    identical in every variant and layout)."""
    rc, p = plan(W, T, H)
    assert rc == A.ARRMS_OK
    assert (p["variant"], p["vec_per_thread"], p["threads_per_row"], p["xcd_chunk"]) == (variant, vpt, tpr, k)


def rplan(W, T, H, lim=LIM, tuning=None, **over):
    b = bufs(W, T, H)
    b.update(over)  # partials / reduced may be given
    return A.arrms_plan_reduce(CU, tuning, lim["max_world"], lim["max_tokens"], lim["max_hidden"], b["partials"], W,
                               T, H, b.get("reduced", b["residual_out"]))


@pytest.mark.parametrize("W,T,H", [(4, 4096, 2048), (8, 16383, 5120), (2, 1, 8), (3, 7, 3), (16, 5, 1000), (11, 3, 2048)])
def test_reduce_plans_cover_every_element(W, T, H):
    rc, p = rplan(W, T, H)
    assert rc == A.ARRMS_OK and p["variant"] == A.ARRMS_VARIANT_REDUCE
    nvec = T * H // 8
    per_block = p["block"] * p["vec_per_thread"]
    assert p["blocks"] == max(1, -(-nvec // per_block)) and p["grid"] == grid_of(p)
    assert p["vec_per_thread"] == 1


@pytest.mark.parametrize("part_off,out_off,elems", [
    (0, 0, 8), (2, 2, 8), (14, 14, 8), (8, 8, 8),      # the same offset everywhere: 16-byte loads after a head
    (0, 8, 4), (8, 0, 4), (0, 4, 2), (4, 12, 4), (0, 2, 1), (6, 0, 1), (2, 10, 4),
])
def test_reduce_load_width(part_off, out_off, elems):
    """The rank sum is flat: the widest load at which every pointer has the same offset."""
    b = bufs(4, 16, 2048)
    parts = [p + part_off for p in b["partials"]]
    rc, p = rplan(4, 16, 2048, partials=parts, reduced=b["residual_out"] + out_off)
    assert rc == A.ARRMS_OK and p["elems_per_load"] == elems
    assert p["variant"] == (A.ARRMS_VARIANT_REDUCE if elems == 8 else A.ARRMS_VARIANT_REDUCE_SCALAR)
    assert p["vec_per_thread"] == (1 if elems == 8 else 0)


def test_reduce_load_width_tuning():
    b = bufs(4, 16, 2048)
    for cap in (1, 2, 4):
        rc, p = A.arrms_plan_reduce(CU, A.arrms_tuning_t.make(scalar_elems=cap), 16, 20000, 65536, b["partials"], 4,
                                    16, 2048, b["residual_out"])
        assert rc == A.ARRMS_OK and p["elems_per_load"] == cap and p["variant"] == A.ARRMS_VARIANT_REDUCE_SCALAR


def test_reduce_plan_validation():
    b = bufs(4, 16, 2048)
    assert rplan(4, 16, 2048, reduced=b["residual"] + 2)[1]["variant"] == A.ARRMS_VARIANT_REDUCE_SCALAR
    assert rplan(4, 16, 2048, reduced=b["partials"][1])[0] == A.ARRMS_OK              # in place into one partial
    assert rplan(4, 16, 2048, reduced=b["partials"][1] + 64)[0] == A.ARRMS_ERR_INVALID_ARG
    assert rplan(4, 16, 2048, reduced=0)[0] == A.ARRMS_ERR_INVALID_ARG
    assert rplan(4, 16, 2048, reduced=b["residual"] + 1)[0] == A.ARRMS_ERR_INVALID_ARG
    assert rplan(17, 16, 2048)[0] == A.ARRMS_ERR_INVALID_ARG
    assert rplan(4, 20001, 2048)[0] == A.ARRMS_ERR_INVALID_ARG
    rc, p = A.arrms_plan_reduce(CU, None, 4, 10, 2048, None, 4, 0, 2048, 0)
    assert rc == A.ARRMS_OK and p["grid"] == 0
    assert A.arrms_reduce(None, b["partials"], 4, 16, 2048, b["residual_out"], 0) == A.ARRMS_ERR_INVALID_ARG


def test_rows_per_block_tuning():
    rc, p = plan(4, 4096, 2048, tuning=A.arrms_tuning_t.make(rows_per_block=4))
    assert rc == A.ARRMS_OK and p["rows_per_block"] == 4 and p["block"] == 1024 and p["blocks"] == 1024
    rc, p = plan(4, 4096, 2048, variant=A.ARRMS_VARIANT_ROW, tuning=A.arrms_tuning_t.make(rows_per_block=8))
    assert rc == A.ARRMS_ERR_UNSUPPORTED                      # 2048 threads per workgroup


@pytest.mark.parametrize("H,offset,elems", [
    (2044, 0, 4), (5122, 0, 2), (1001, 0, 1), (2046, 0, 2),            # H decides
    (2048, 8, 4), (2048, 4, 2), (2048, 2, 1), (2044, 4, 2), (5122, 2, 1),  # a pointer's alignment decides
])
@pytest.mark.parametrize("field", ["residual", "weight", "norm_out", "partial"])
def test_scalar_load_width(H, offset, elems, field):
    """The widest load (in BF16 elements) that H and every pointer's alignment allow."""
    b = bufs(4, 64, H)
    if offset:
        if field == "partial":
            b["partials"][2] += offset
        else:
            b[field] += offset
    rc, p = plan(4, 64, H, **b)
    assert rc == A.ARRMS_OK and p["variant"] == A.ARRMS_VARIANT_SCALAR
    assert p["elems_per_load"] == elems and p["vec_per_thread"] == 0


def test_scalar_load_width_tuning_and_vector_plans():
    rc, p = plan(4, 64, 2044, tuning=A.arrms_tuning_t.make(scalar_elems=1))
    assert p["elems_per_load"] == 1
    rc, p = plan(4, 64, 5122, tuning=A.arrms_tuning_t.make(scalar_elems=4))   # capped by H
    assert p["elems_per_load"] == 2
    rc, p = plan(4, 64, 2048, variant=A.ARRMS_VARIANT_SCALAR)                # forced: widest allowed
    assert p["elems_per_load"] == 4 and p["block"] == 256
    rc, p = plan(4, 64, 2048)
    assert p["variant"] == A.ARRMS_VARIANT_ROW and p["elems_per_load"] == 0
    assert plan(4, 64, 2044, tuning=A.arrms_tuning_t.make(scalar_elems=3))[0] == A.ARRMS_ERR_INVALID_ARG


# residual_out store policy: the row and scalar kernels stream it (non-temporal stores)
# unless tuned; split-H always writes it back (its second kernel reads residual_out again).
@pytest.mark.parametrize("W,T,H,variant,cached", [
    (4, 4096, 2048, A.ARRMS_VARIANT_ROW, 0),
    (2, 6144, 2048, A.ARRMS_VARIANT_ROW, 0),
    (8, 16383, 5120, A.ARRMS_VARIANT_ROW, 0),
    (4, 4096, 2047, A.ARRMS_VARIANT_SCALAR, 0),
    (8, 16383, 5119, A.ARRMS_VARIANT_SCALAR, 0),
    (8, 1, 8192, A.ARRMS_VARIANT_SPLITH, 1),
    (4, 16, 16384, A.ARRMS_VARIANT_SPLITH, 1),
])
def test_residual_out_store_policy(W, T, H, variant, cached):
    rc, p = plan(W, T, H)
    assert rc == A.ARRMS_OK and p["variant"] == variant, p
    assert p["residual_out_cached"] == cached


# More than 8 ranks: the automatic choice takes the scalar kernel for rows of at most 8192
# elements from 4 rows per CU (8 at W=16); fewer rows, longer rows, at most 5 ranks or a
# tuned lane layout keep their plans.
@pytest.mark.parametrize("W,T,H,variant", [
    (12, 1024, 4096, A.ARRMS_VARIANT_SCALAR), (12, 1023, 4096, A.ARRMS_VARIANT_ROW),
    (9, 1024, 2048, A.ARRMS_VARIANT_SCALAR), (15, 4096, 2048, A.ARRMS_VARIANT_SCALAR),
    (16, 2048, 2048, A.ARRMS_VARIANT_SCALAR), (16, 2047, 2048, A.ARRMS_VARIANT_ROW),
    (16, 4096, 4104, A.ARRMS_VARIANT_SCALAR), (5, 16384, 2048, A.ARRMS_VARIANT_ROW),
    (12, 4096, 8192, A.ARRMS_VARIANT_SCALAR), (12, 4096, 8200, A.ARRMS_VARIANT_SPLITH),
    (10, 1024, 2560, A.ARRMS_VARIANT_SCALAR),
])
def test_many_ranks_take_the_scalar_kernel(W, T, H, variant):
    rc, p = plan(W, T, H)
    assert rc == A.ARRMS_OK and p["variant"] == variant, (W, T, H, p)
    if variant == A.ARRMS_VARIANT_SCALAR:
        assert p["elems_per_load"] == (4 if H % 4 == 0 else 2)


# Six to eight ranks: the scalar kernel's rank loop on power-of-two workgroups (H rounding
# up to 256, 512 or 1024 lanes) from 8 rows per CU; other lane counts keep the row kernel.
@pytest.mark.parametrize("W,T,H,loop", [
    (8, 8192, 8192, True), (8, 2048, 2048, True), (8, 2047, 2048, False), (6, 4096, 4096, True),
    (7, 4096, 8192, True), (8, 16383, 5120, False), (8, 4096, 3072, False), (5, 4096, 8192, False),
    (8, 4096, 2040, True), (8, 4096, 7168, False),
])
def test_mid_ranks_rank_loop(W, T, H, loop):
    rc, p = plan(W, T, H)
    assert rc == A.ARRMS_OK
    if loop:
        assert p["variant"] == A.ARRMS_VARIANT_SCALAR and p["rank_loop"] == 1 and p["block"] in (256, 512, 1024), p
    else:
        assert p["variant"] == A.ARRMS_VARIANT_ROW and p["rank_loop"] == 0, p
    t = A.arrms_tuning_t.make(vec_per_thread=1 if H <= 4096 else 2)   # a tuned layout keeps the row kernel
    assert plan(W, T, H, tuning=t)[1]["variant"] == A.ARRMS_VARIANT_ROW


# Rows whose stride is not a multiple of 128 bytes (H % 64 != 0): the scalar kernel
# (8-byte loads, lanes rotated onto whole lines) for rows of 256-1024 lanes from 16 rows
# per CU, and for shorter rows at one rank from 64 rows per CU; aligned strides, longer
# rows, fewer rows and tuned lane layouts keep the row kernel.
@pytest.mark.parametrize("W,T,H,variant", [
    (4, 4096, 2040, A.ARRMS_VARIANT_SCALAR), (4, 4095, 2040, A.ARRMS_VARIANT_ROW),
    (4, 4096, 2048, A.ARRMS_VARIANT_ROW), (1, 4096, 2040, A.ARRMS_VARIANT_SCALAR),
    (2, 16384, 6000, A.ARRMS_VARIANT_SCALAR), (4, 4096, 8136, A.ARRMS_VARIANT_SCALAR),
    (4, 4096, 8200, A.ARRMS_VARIANT_ROW), (5, 8192, 1544, A.ARRMS_VARIANT_SCALAR),
    (4, 16384, 1528, A.ARRMS_VARIANT_ROW), (4, 16384, 520, A.ARRMS_VARIANT_ROW),
    (1, 16384, 1000, A.ARRMS_VARIANT_SCALAR), (1, 16383, 1000, A.ARRMS_VARIANT_ROW),
    (2, 16384, 1000, A.ARRMS_VARIANT_ROW), (8, 8192, 3000, A.ARRMS_VARIANT_SCALAR),
])
def test_line_offset_rows_take_the_scalar_kernel(W, T, H, variant):
    rc, p = plan(W, T, H)
    assert rc == A.ARRMS_OK and p["variant"] == variant, (W, T, H, p)
    if variant == A.ARRMS_VARIANT_SCALAR:
        assert p["elems_per_load"] == 4 and p["rank_loop"] == 0, p
    for t in (dict(vec_per_thread=1), dict(threads_per_row=256), dict(rows_per_block=1)):
        rc, p = plan(W, T, H, tuning=A.arrms_tuning_t.make(**t))
        assert rc == A.ARRMS_OK and p["variant"] == A.ARRMS_VARIANT_ROW or H > 8192, (t, p)
    rc, p = plan(4, 2048, 2040, cu=128)                           # 16 rows per CU on 128 CUs
    assert p["variant"] == A.ARRMS_VARIANT_SCALAR


# Preloaded kernel arguments: the flat-argument twins serve row, scalar (without the rank
# loop) and rank-sum calls with W <= 8 from 16 MiB of traffic per call; tuning turns
# them off (1) or on wherever a twin exists (2).
@pytest.mark.parametrize("W,T,H,want", [
    (4, 4096, 2048, 1), (4, 585, 2048, 1), (4, 584, 2048, 0), (4, 1, 2048, 0), (8, 16383, 5120, 1),
    (8, 8192, 8192, 0), (4, 4096, 2047, 1), (12, 4096, 2048, 0), (8, 1, 8192, 0), (1, 16384, 512, 1),
    (4, 4096, 2040, 1), (8, 4096, 4095, 0), (7, 4096, 4095, 1),
])
def test_kernarg_preload_plan(W, T, H, want):
    rc, p = plan(W, T, H)
    assert rc == A.ARRMS_OK and p["kernarg_preload"] == want, (W, T, H, p)
    twin = W <= 8 and (p["variant"] == A.ARRMS_VARIANT_ROW or
                       (p["variant"] == A.ARRMS_VARIANT_SCALAR and not p["rank_loop"]))
    assert plan(W, T, H, tuning=A.arrms_tuning_t.make(kernarg_preload=1))[1]["kernarg_preload"] == 0
    assert plan(W, T, H, tuning=A.arrms_tuning_t.make(kernarg_preload=2))[1]["kernarg_preload"] == int(twin)
    assert 2 * T * H * (W + 3) + 2 * H >= 16 << 20 or not want


def test_kernarg_preload_reduce_plan():
    for W, T, want in ((4, 4096, 1), (2, 16, 0), (8, 16384, 0), (5, 16384, 1), (12, 4096, 0)):
        rc, p = rplan(W, T, 2048)
        assert rc == A.ARRMS_OK and p["kernarg_preload"] == want, (W, T, p)
    assert rplan(4, 4096, 2048, tuning=A.arrms_tuning_t.make(kernarg_preload=1))[1]["kernarg_preload"] == 0
    assert rplan(2, 16, 2048, tuning=A.arrms_tuning_t.make(kernarg_preload=2))[1]["kernarg_preload"] == 1
    assert rplan(8, 16384, 2048, tuning=A.arrms_tuning_t.make(kernarg_preload=2))[1]["kernarg_preload"] == 0


def test_kernarg_preload_tuning_range():
    for bad in (-1, 3):
        rc, _ = plan(4, 4096, 2048, tuning=A.arrms_tuning_t.make(kernarg_preload=bad))
        assert rc == A.ARRMS_ERR_INVALID_ARG


def test_many_ranks_rule_scales_with_cus_and_respects_tuning():
    lim = dict(LIM)
    rc, p = plan(12, 512, 2048, cu=128, lim=lim)                # 4 rows per CU on 128 CUs
    assert p["variant"] == A.ARRMS_VARIANT_SCALAR
    rc, p = plan(12, 511, 2048, cu=128, lim=lim)
    assert p["variant"] == A.ARRMS_VARIANT_ROW
    for t in (dict(vec_per_thread=1), dict(threads_per_row=256), dict(rows_per_block=1)):
        rc, p = plan(12, 4096, 2048, tuning=A.arrms_tuning_t.make(**t))
        assert rc == A.ARRMS_OK and p["variant"] == A.ARRMS_VARIANT_ROW, t


@pytest.mark.parametrize("W,T,loop", [(12, 2048, 1), (12, 2047, 0), (16, 4096, 1), (9, 2048, 1), (8, 16384, 1),
                                       (6, 2048, 1), (5, 16384, 0), (4, 16384, 0), (16, 1024, 0), (16, 256, 0)])
def test_reduce_rank_loop(W, T, loop):
    """Six ranks or more: the rank sum adds them one load round at a time from 8
    workgroups per CU (2048 elements per workgroup: T*H >= 8 * 256 * 2048)."""
    rc, p = rplan(W, T, 2048)
    assert rc == A.ARRMS_OK and p["rank_loop"] == loop, p
    assert p["blocks"] == T * 2048 // 2048


def test_scalar_rank_loop_flag():
    assert plan(12, 64, 2047)[1]["rank_loop"] == 1 and plan(8, 64, 2047)[1]["rank_loop"] == 0
    assert plan(16, 4096, 2048)[1]["rank_loop"] == 1                     # the many-ranks scalar plan
    assert plan(16, 33, 2048)[1]["rank_loop"] == 0                       # row kernel
    assert plan(8, 4096, 2047)[1]["rank_loop"] == 0                      # odd rows on 256 lanes: specialised
    # odd rows with eight ranks on 512 lanes or more, 8 rows per CU: the rank loop
    for W, T, H, want in ((8, 4096, 4095, 1), (8, 2048, 5119, 1), (8, 2047, 5119, 0), (7, 4096, 4095, 0),
                          (8, 4096, 8191, 1), (8, 4096, 9001, 0)):
        rc, p = plan(W, T, H)
        assert rc == A.ARRMS_OK and p["variant"] == A.ARRMS_VARIANT_SCALAR and p["rank_loop"] == want, (W, T, H, p)
    t = A.arrms_tuning_t.make(scalar_elems=1)
    assert plan(8, 4096, 4095, tuning=t)[1]["rank_loop"] == 0


def test_scalar_lanes_tuning():
    """threads_per_row sets the scalar kernel's lanes per row when it is a multiple of 64."""
    for tpr, want in ((256, 256), (512, 512), (64, 64), (1024, 1024), (32, 640)):
        rc, p = plan(8, 100, 5119, tuning=A.arrms_tuning_t.make(threads_per_row=tpr))
        assert rc == A.ARRMS_OK and p["variant"] == A.ARRMS_VARIANT_SCALAR and p["block"] == want, (tpr, p)
    rc, p = plan(12, 100, 5119, tuning=A.arrms_tuning_t.make(threads_per_row=1024))   # any rank count: up to 1024
    assert p["block"] == 1024


def test_residual_out_store_tuning():
    for store, want in ((1, 0), (2, 1)):
        t = A.arrms_tuning_t.make(residual_out_store=store)
        for W, T, H in ((4, 4096, 2048), (8, 16383, 5120), (4, 64, 2047), (2, 16, 2048)):
            rc, p = plan(W, T, H, tuning=t)
            assert rc == A.ARRMS_OK and p["residual_out_cached"] == want, (W, T, H, p)
        rc, p = plan(8, 1, 8192, tuning=t)                        # split-H reads it back: always write-back
        assert p["variant"] == A.ARRMS_VARIANT_SPLITH and p["residual_out_cached"] == 1
    for bad in (-1, 3):
        assert plan(4, 64, 2048, tuning=A.arrms_tuning_t.make(residual_out_store=bad))[0] == A.ARRMS_ERR_INVALID_ARG
    rc, p = rplan(4, 16, 2048)
    assert rc == A.ARRMS_OK and p["residual_out_cached"] == 0    # the rank sum writes no residual_out


def test_tuned_rows_per_block_keeps_one_vector_layout():
    """Tuning only the rows per workgroup is a layout override: the automatic four-vector
    layout (16 lanes per row at H=512) is not taken, so the row kernel still runs."""
    rc, p = plan(1, 16384, 512, tuning=A.arrms_tuning_t.make(rows_per_block=1))
    assert rc == A.ARRMS_OK
    assert (p["variant"], p["vec_per_thread"], p["threads_per_row"], p["rows_per_block"]) == (
        A.ARRMS_VARIANT_ROW, 1, 64, 1)


@pytest.mark.parametrize("tuning", [dict(vec_per_thread=4), dict(vec_per_thread=8), dict(splith_block=64)])
def test_automatic_choice_never_fails_under_tuning(tuning):
    """Tuning changes speed only: where no vector kernel can honour it, the automatic
    choice ends in the scalar kernel instead of refusing the call."""
    for W, T, H in ((4, 3, 32768), (4, 5000, 65536), (8, 2, 8192), (4, 4096, 2048)):
        rc, p = plan(W, T, H, tuning=A.arrms_tuning_t.make(**tuning))
        assert rc == A.ARRMS_OK, (W, T, H, tuning)
        assert p["variant"] in (A.ARRMS_VARIANT_ROW, A.ARRMS_VARIANT_SPLITH, A.ARRMS_VARIANT_SCALAR)
        assert p["grid"] > 0


@pytest.mark.parametrize("W,T,H,variant", [
    (8, 1, 5120, A.ARRMS_VARIANT_ROW),          # 110 KiB per row: below 144 KiB, never split
    (4, 1, 8192, A.ARRMS_VARIANT_ROW),          # 112 KiB
    (2, 1, 12288, A.ARRMS_VARIANT_ROW),         # 120 KiB
    (8, 1, 6144, A.ARRMS_VARIANT_ROW),          # 132 KiB
    (8, 96, 8192, A.ARRMS_VARIANT_SPLITH),      # 176 KiB: split up to 64 * 48 / 32 = 96 rows
    (8, 97, 8192, A.ARRMS_VARIANT_ROW),
    (4, 128, 16384, A.ARRMS_VARIANT_SPLITH),    # 224 KiB: 192 by the slope, capped at 128
    (4, 129, 16384, A.ARRMS_VARIANT_ROW),
    (16, 48, 4096, A.ARRMS_VARIANT_SPLITH),     # 152 KiB: 64 * 24 / 32 = 48 rows
    (16, 49, 4096, A.ARRMS_VARIANT_ROW),
    (16, 129, 6144, A.ARRMS_VARIANT_SPLITH),    # the row kernels cannot hold this row at W=16
])
def test_splith_crossover_boundaries(W, T, H, variant):
    """The automatic split-H rule with 256 CUs: rows of 144 KiB or more split while
    T <= 64 * (row KiB - 128) / 32, at most 128 rows."""
    rc, p = plan(W, T, H)
    assert rc == A.ARRMS_OK and p["variant"] == variant, (W, T, H, p)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback: with the library missing every entry point raises."""
    import subprocess
    import sys
    code = ("import residual_add_rmsnorm_arrms_amd as A; A.LIB_PATH = %r\n"
            "try:\n    A.arrms_status_string(0)\nexcept RuntimeError as e:\n    print('raised', 'not built' in str(e))\n"
            % str(tmp_path / "missing.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.check_output([sys.executable, "-c", code], cwd=root, env=dict(os.environ, PYTHONPATH=root))
    assert out.decode().strip() == "raised True"


def test_operator_checks_tensor_arguments():
    import torch
    op = A.FusedReduceResidualRMSNorm.__new__(A.FusedReduceResidualRMSNorm)  # no handle needed for the checks
    x = torch.zeros((2, 4, 16), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        op._args(x, torch.zeros((4, 16), dtype=torch.bfloat16), torch.zeros(16, dtype=torch.bfloat16), None, None)


def test_fused_noalloc_wrapper_needs_both_outputs():
    """The torch-level no-allocation call allocates nothing, so it refuses missing outputs
    before touching any device."""
    import torch
    x = torch.zeros((2, 4, 16), dtype=torch.bfloat16)
    r = torch.zeros((4, 16), dtype=torch.bfloat16)
    w = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="allocates nothing"):
        A.fused_noalloc(x, r, w, 1e-6, None, torch.zeros_like(r))
    with pytest.raises(ValueError, match="allocates nothing"):
        A.fused_noalloc(x, r, w, 1e-6, torch.zeros_like(r), None)
