"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only, g++/gcc):
the library's validation and planning (arrms_plan, arrms_plan_reduce) fuzzed with
random arguments, and the CPU oracle on random shapes and bit patterns."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ROCM = "/opt/rocm"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_fuzz")
    _run(["gcc", *SAN, "-std=c99", "-fno-fast-math", "-ffp-contract=off",
          os.path.join(ROOT, "tests", "sanitize", "oracle_fuzz.c"), os.path.join(ROOT, "oracle", "arrms_oracle.c"),
          "-o", exe, "-lm"])
    assert "oracle fuzz ok" in _run([exe])


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")),
                    reason="HIP headers not installed")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    csrc = os.path.join(ROOT, "residual_add_rmsnorm_arrms_amd", "csrc")
    _run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", csrc,
          "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "sanitize", "plan_fuzz.cpp"),
          os.path.join(csrc, "arrms_api.cpp"), "-o", exe, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    assert "plan fuzz ok" in _run([exe, "200000"], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
