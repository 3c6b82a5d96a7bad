"""Write tests/golden/frozen_*.txt: the oracle's outputs on small seeded workloads,
frozen so that a later change to the oracle, to the input generator or to the
GPU path shows up as a diff against fixed bits.

Calls only oracle/ and synth/ (the seeded generator): python tests/golden/make_frozen.py
Each file holds, per workload: its parameters, then one line per token row with the
residual_out and norm_out BF16 bit patterns in hex, and the row's binary32 1/RMS
bit pattern.  The values come from the oracle; what pins the oracle itself is the
rest of tests/oracle_pins.py (hand-derived rows, exact-arithmetic emulation,
invariants), not this file.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

# name -> workload (small enough to store; they span a ragged H, W = 1 and W = 16)
FROZEN = {
    "tiny": synth.WORKLOADS["tiny"],
    "w3_h136": synth.Workload("w3_h136", world=3, tokens=5, hidden=136, seed=11),
    "w1_h64_eps0": synth.Workload("w1_h64_eps0", world=1, tokens=3, hidden=64, eps=0.0, seed=12),
    "w16_h40_outliers": synth.Workload("w16_h40_outliers", world=16, tokens=4, hidden=40, outlier_p=0.05, seed=13),
}


def render(wl) -> str:
    x, r, w = synth.make_inputs(wl)
    out = oracle.fused(synth.bits(x), synth.bits(r), synth.bits(w), wl.eps)
    lines = ["workload %s W %d T %d H %d seed %d x_sigma %r eps %r outlier_p %r" % (
        wl.name, wl.world, wl.tokens, wl.hidden, wl.seed, wl.x_sigma, wl.eps, wl.outlier_p)]
    for t in range(wl.tokens):
        ro = " ".join("%04x" % v for v in out["residual_out"][t])
        no = " ".join("%04x" % v for v in out["norm_out"][t])
        inv = "%08x" % int(out["inv_rms"][t:t + 1].view(np.uint32)[0])
        lines.append("row %d inv %s" % (t, inv))
        lines.append("ro " + ro)
        lines.append("no " + no)
    return "\n".join(lines) + "\n"


def path(name) -> str:
    return os.path.join(HERE, "frozen_%s.txt" % name)


if __name__ == "__main__":
    for name, wl in FROZEN.items():
        with open(path(name), "w") as f:
            f.write(render(wl))
        print("wrote", path(name))
