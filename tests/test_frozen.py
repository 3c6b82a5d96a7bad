"""Frozen outputs (tests/golden/frozen_*.txt, written by tests/golden/make_frozen.py
from the oracle): the oracle and the seeded generator must still reproduce them bit
for bit (CPU), and the GPU library must match them to the parity bar (GPU)."""
import numpy as np
import pytest

import synth
from tests.golden import make_frozen

NAMES = sorted(make_frozen.FROZEN)


def parse(name):
    rows = {"inv": [], "ro": [], "no": []}
    for line in open(make_frozen.path(name)):
        key, _, rest = line.strip().partition(" ")
        if key == "row":
            rows["inv"].append(int(rest.split()[-1], 16))
        elif key in ("ro", "no"):
            rows[key].append([int(v, 16) for v in rest.split()])
    return (np.array(rows["ro"], dtype=np.uint16), np.array(rows["no"], dtype=np.uint16),
            np.array(rows["inv"], dtype=np.uint32))


@pytest.mark.parametrize("name", NAMES)
def test_oracle_and_generator_reproduce_the_frozen_file(name):
    assert make_frozen.render(make_frozen.FROZEN[name]) == open(make_frozen.path(name)).read()


@pytest.mark.gpu
@pytest.mark.parametrize("name", NAMES)
def test_gpu_matches_the_frozen_file(name):
    import torch

    from tests.gpu_util import assert_parity, run, say
    wl = make_frozen.FROZEN[name]
    say("case frozen %s" % name)
    x, r, w = synth.make_inputs(wl)
    ro, no, plan = run(x, r, w, wl.eps)
    want_ro, want_no, _ = parse(name)
    assert_parity(ro, no, {"residual_out": want_ro, "norm_out": want_no}, "frozen " + name)
    torch.cuda.synchronize()
