"""The boundary from plain C: tests/abi_c/plan_demo.c includes include/arrms.h, is
compiled by gcc as C99 with warnings as errors, links libarrms.so and exercises the
host-only entry points (planning, validation, status strings, null-handle calls).
No GPU is needed."""
import os
import shutil
import subprocess

import pytest

import residual_add_rmsnorm_arrms_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE), reason="needs gcc and ROCm headers")
def test_c_caller_compiles_links_and_runs(tmp_path):
    if not os.path.exists(A.LIB_PATH):
        from residual_add_rmsnorm_arrms_amd import build
        build.build()
    exe = str(tmp_path / "plan_demo")
    libdir = os.path.dirname(A.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "abi_c", "plan_demo.c"), "-o", exe,
           "-L", libdir, "-larrms", "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "FAIL" not in res.stdout and res.stdout.count("ok   ") == 9, res.stdout
