"""Build ``libarrms.so`` (the gfx950 HIP library) in place with hipcc.

The library is always compiled for gfx950 only.  Floating-point flags keep the
kernels' arithmetic plain IEEE: no fast-math, no FMA contraction, binary32
denormals kept, and packed binary32 instructions disabled.  Kernel arguments passed
as a flat list of scalars are preloaded into scalar registers.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libarrms.so")
SOURCES = [os.path.join(CSRC, "arrms_kernels.hip"), os.path.join(CSRC, "arrms_reduce.hip"),
           os.path.join(CSRC, "arrms_api.cpp"), os.path.join(CSRC, "arrms_noalloc.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    # kernels whose arguments are a flat list of scalars get the leading 14 dwords
    # preloaded into scalar registers at wave launch (a no-op for by-value blocks)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def build(verbose: bool = False) -> str:
    """Compile the library (always, even when one exists) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-Wl,-soname,libarrms.so", "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so; that is harmless.
    noise = ("packed-fp32-ops", "not a recognized feature", "warning generated", "warnings generated")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
