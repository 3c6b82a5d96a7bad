"""The seeded input generator: deterministic, thread-count independent, right distributions."""
import os
import subprocess
import sys

import numpy as np
import pytest

import synth
from tests.bf16util import bf16_values


def test_same_seed_same_bytes_and_streams_differ():
    a = synth.normal_f32(0, 1, 1.0, 10001)
    b = synth.normal_f32(0, 1, 1.0, 10001)
    c = synth.normal_f32(0, 2, 1.0, 10001)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)
    # prefix property of a counter-based stream
    np.testing.assert_array_equal(synth.normal_f32(0, 1, 1.0, 100), a[:100])


def test_bytes_do_not_depend_on_thread_count():
    code = ("import synth, numpy as np, sys; a = synth.normal_f32(0, 5, 1.0, 200001, 0.01, 100.0, 7);"
            "sys.stdout.write(str(int(np.frombuffer(a.tobytes(), np.uint32).astype(np.uint64).sum())))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = set()
    for n in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=n, PYTHONPATH=root)
        outs.add(subprocess.check_output([sys.executable, "-c", code], env=env, cwd=root))
    assert len(outs) == 1


def test_distributions():
    n = 400000
    a = synth.normal_f32(0, 3, 0.5, n).astype(np.float64)
    assert abs(a.mean()) < 0.005 and abs(a.std() - 0.5) < 0.005
    u = synth.uniform_f32(0, 4, 0.5, 1.5, n).astype(np.float64)
    assert u.min() >= 0.5 and u.max() <= 1.5 and abs(u.mean() - 1.0) < 0.005
    o = synth.normal_f32(0, 3, 0.5, n, 0.01, 100.0, 9).astype(np.float64)
    frac = np.mean(o != a)
    assert 0.009 < frac < 0.011
    np.testing.assert_allclose(o[o != a], a[o != a] * 100.0, rtol=1e-6)


def test_workload_shapes_and_dtype():
    wl = synth.WORKLOADS["tiny"]
    x, res, w = synth.make_inputs(wl)
    assert tuple(x.shape) == (2, 4, 128) and tuple(res.shape) == (4, 128) and tuple(w.shape) == (128,)
    wv = bf16_values(synth.bits(w))
    assert wv.min() >= 0.5 and wv.max() <= 1.5
    assert wl.algorithmic_bytes == 2 * 4 * 128 * 5 + 2 * 128
    assert synth.WORKLOADS["prefill"].algorithmic_bytes == 117444608
