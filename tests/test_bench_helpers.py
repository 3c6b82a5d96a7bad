"""Host-side pieces of bench.py: the algorithmic byte count, percentiles, the kernel
source hash that keys the traffic record (comments do not change it, code does), and
the refusal of more than one GPU."""
import subprocess
import sys

import bench


def test_algorithmic_bytes():
    # read W partials + residual, write two outputs, read the weight once
    assert bench.algorithmic_bytes(4, 4096, 2048) == 2 * 4096 * 2048 * 7 + 2 * 2048 == 117444608
    assert bench.algorithmic_bytes(1, 1, 8) == 2 * 8 * 4 + 16


def test_percentiles():
    xs = list(range(101))
    assert bench.pct(xs, 50) == 50 and bench.pct(xs, 90) == 90 and bench.pct(xs, 99) == 99
    assert bench.pct([3.0], 99) == 3.0


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("int f() {\n    return 1;  // one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", [str(a)])
    h1 = bench.kernel_source_hash()
    a.write_text("// a new comment\nint f() {\n    return 1;  // changed comment\n}\n\n")
    assert bench.kernel_source_hash() == h1
    a.write_text("int f() {\n    return 2;\n}\n")
    assert bench.kernel_source_hash() != h1


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr and res.stdout == ""


def test_source_hash_covers_planner_and_argument_packing():
    """A planner or argument-layout change re-keys the traffic record like a kernel change."""
    names = sorted(p.rsplit("/", 1)[-1] for p in bench.KERNEL_SRC)
    assert names == ["arrms_api.cpp", "arrms_device.h", "arrms_internal.h", "arrms_kernels.hip"]


def test_traffic_record_needs_same_source_and_plan(tmp_path, monkeypatch):
    import json
    import synth
    wl = synth.WORKLOADS["prefill"]
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(tmp_path / "t.json"))
    plan = {"grid": 4096, "block": 256, "xcd_chunk": 64}
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "plan": plan, "read_bytes_per_launch": 1.0,
           "write_bytes_per_launch": 2.0}
    json.dump(rec, open(tmp_path / "t.json", "w"))
    assert bench.traffic_record(wl, plan)["write_bytes_per_launch"] == 2.0
    assert bench.traffic_record(wl, dict(plan, xcd_chunk=32)) is None       # another launch plan
    json.dump(dict(rec, kernel_source_sha256_16="0" * 16), open(tmp_path / "t.json", "w"))
    assert bench.traffic_record(wl, plan) is None                           # other source


def _args(**kw):
    import argparse
    d = dict(workload="prefill", world=None, tokens=None, hidden=None, eps=None, x_sigma=None, outlier_p=None,
             seed=None)
    d.update(kw)
    return argparse.Namespace(**d)


def test_custom_shape_arguments():
    import pytest
    import synth
    assert bench.workload_from_args(synth, _args()) is synth.WORKLOADS["prefill"]
    wl = bench.workload_from_args(synth, _args(world=8, tokens=1000, hidden=5120, eps=1e-5, x_sigma=2.0))
    assert (wl.name, wl.world, wl.tokens, wl.hidden, wl.eps, wl.x_sigma) == ("custom", 8, 1000, 5120, 1e-5, 2.0)
    assert wl.residual_sigma == 1.0 and wl.weight_lo == 0.5 and wl.outlier_p == 0.0   # the rest from prefill
    assert wl.algorithmic_bytes == bench.algorithmic_bytes(8, 1000, 5120) == 2 * 1000 * 5120 * 11 + 2 * 5120
    wl = bench.workload_from_args(synth, _args(workload="ragged_outliers", tokens=17))
    assert wl.outlier_p == 0.01 and wl.world == 8 and wl.tokens == 17
    for bad in (dict(world=17), dict(world=0), dict(tokens=0), dict(hidden=65537), dict(eps=-1.0),
                dict(outlier_p=1.5), dict(x_sigma=0.0)):
        with pytest.raises(SystemExit):
            bench.workload_from_args(synth, _args(**bad))


def test_pool_slots_fit_the_gpu():
    import types
    import pytest
    gib = 2 ** 30
    fake = types.SimpleNamespace(cuda=types.SimpleNamespace(
        get_device_properties=lambda i: types.SimpleNamespace(total_memory=288 * gib)))
    assert bench.pool_slots(fake, 0.44 * gib) == 10        # the prefill pool's slot
    assert bench.pool_slots(fake, 30 * gib) == 4           # 4 x 30 GiB within half of 288 GiB
    with pytest.raises(SystemExit):
        bench.pool_slots(fake, 100 * gib)


def test_custom_shape_on_the_command_line_is_checked_before_the_gpu():
    res = subprocess.run([sys.executable, bench.__file__, "--world", "40"], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode != 0 and "out of range" in res.stderr and res.stdout == ""
