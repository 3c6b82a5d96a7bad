"""The oracle pins are sharp: each plausible mistake, planted in a copy of the oracle's
C source on the CPU, fails at least one pin of tests/oracle_pins.py.

Each mutant is one textual edit of oracle/arrms_oracle.c, compiled into a temporary
library with the oracle's own gcc flags; the real oracle is never modified.
"""
import os
import tempfile

import pytest

import oracle
from tests.oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "arrms_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("rank_sum_reverse_order",
     "float acc = widen(x[0][row + h]);\n            for (int r = 1; r < W; ++r) acc = acc + widen(x[r][row + h]);",
     "float acc = widen(x[W - 1][row + h]);\n            for (int r = W - 2; r >= 0; --r) acc = acc + widen(x[r][row + h]);"),
    ("rank_sum_drops_last_rank", "for (int r = 1; r < W; ++r)", "for (int r = 1; r < W - 1; ++r)"),
    ("rank_sum_sign", "acc = acc + widen(x[r]", "acc = acc - widen(x[r]"),
    ("reduced_not_rounded", "round_bf16(widen(red) + widen(residual[row + h]))",
     "round_bf16(acc + widen(residual[row + h]))"),
    ("residual_dropped", "round_bf16(widen(red) + widen(residual[row + h]))", "round_bf16(widen(red))"),
    ("residual_wrong_row", "widen(residual[row + h])", "widen(residual[h])"),
    ("eps_outside_root", "1.0 / sqrt(mean_sq + (double)eps)", "1.0 / (sqrt(mean_sq) + (double)eps)"),
    ("eps_dropped", "1.0 / sqrt(mean_sq + (double)eps)", "1.0 / sqrt(mean_sq)"),
    ("sum_not_mean", "sum_sq / (double)H", "sum_sq"),
    ("mean_over_h_minus_1", "sum_sq / (double)H", "sum_sq / (double)(H - 1)"),
    ("sum_sq_in_binary32", "double sum_sq = 0.0;", "float sum_sq = 0.0f;"),
    ("square_of_unrounded_sum", "const double v = (double)widen(ro);", "const double v = (double)(widen(red) + widen(residual[row + h]));"),
    ("weight_reversed", "widen(weight[h])", "widen(weight[H - 1 - h])"),
    ("weight_plus_one", "normed * widen(weight[h])", "normed * (1.0f + widen(weight[h]))"),
    ("weight_ignored", "normed * widen(weight[h])", "normed"),
    ("inv_not_applied", "widen(residual_out[row + h]) * inv", "widen(residual_out[row + h])"),
    ("ties_away_from_zero", "(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    ("truncate_not_round", "kept += 1u;", "kept += 0u;"),
    ("nan_not_quieted", "return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);"),
    ("widen_wrong_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("scale_before_normalise",
     "const float normed = widen(residual_out[row + h]) * inv;\n            const float scaled = normed * widen(weight[h]);",
     "const float normed = widen(residual_out[row + h]) * widen(weight[h]);\n            const float scaled = normed * inv;"),
    ("inv_rounded_before_reciprocal", "(float)(1.0 / sqrt(mean_sq + (double)eps))",
     "1.0f / (float)sqrt(mean_sq + (double)eps)"),
    ("rank_sum_in_binary64", "float acc = widen(x[0][row + h]);", "double acc = widen(x[0][row + h]);"),
]


@pytest.fixture(scope="module")
def source():
    return open(SRC).read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new, tmp_path):
    assert source.count(old) >= 1, "mutation site not found: %s" % name
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(source.replace(old, new))
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / ("libmut_%s.so" % name)))
    orc = oracle.Oracle(lib)
    caught = []
    for pin_name, fn, kw in PINS:
        try:
            fn(orc, **kw)
        except AssertionError:
            caught.append(pin_name)
    assert caught, "mutant %s passed every pin" % name
