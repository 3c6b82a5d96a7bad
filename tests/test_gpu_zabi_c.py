"""The boundary from plain C on the GPU (tests/abi_c/fused_demo.c, built by
__graft_entry__.build()): create, fused call on hipMalloc'd buffers, destroy, with the
outputs checked against the oracle inside the C program, then a C loop of
back-to-back calls timed with HIP events (printed); then the no-allocation entry
point, which must give arrms_fused's bits, and its own timed loop."""
import os
import subprocess

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "abi_c", "fused_demo")


@pytest.mark.parametrize("W,T,H,calls", [(4, 37, 2048, 200), (4, 1, 2048, 5000), (4, 16, 2048, 5000),
                                         (4, 4096, 2048, 2000), (8, 64, 5120, 1000), (3, 5, 1001, 200),
                                         (16, 3, 2048, 200)])
def test_c_program_end_to_end(W, T, H, calls):
    if not os.path.exists(DEMO):  # normally built by __graft_entry__.build(); a plain gcc link, about a second
        import __graft_entry__
        __graft_entry__.build_c_demo()
    say("case C program W=%d T=%d H=%d calls=%d" % (W, T, H, calls))
    res = subprocess.run([DEMO, str(W), str(T), str(H), str(calls)], capture_output=True, text=True, timeout=90)
    out = res.stdout + res.stderr
    say(out.strip())
    assert res.returncode == 0, out
    assert "FAIL" not in out and "timing:" in out and "arrms_fused_noalloc outputs bit-identical" in out
