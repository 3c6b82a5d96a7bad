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
