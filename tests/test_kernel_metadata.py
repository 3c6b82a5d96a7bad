"""Code-object properties of the gfx950 kernels, read from the metadata hipcc emits
for this repository's own sources (compiled here with the library's flags):

- no kernel spills registers or uses private (scratch) memory;
- no kernel needs the implicit-argument block (no blockDim / gridDim reads);
- every kernel specialised on W <= 8 (and the W-independent ones) takes at most
  112 bytes of arguments: on MI355X with ROCm 7 the host cost of a launch steps
  up by about 0.9 us beyond that, which matters for decode-sized calls.
"""
import os
import re
import subprocess

import pytest
import yaml

from residual_add_rmsnorm_arrms_amd import build as B

SOURCES = [os.path.join(B.CSRC, f) for f in ("arrms_kernels.hip", "arrms_reduce.hip")]
MAX_FAST_ARGS = 112


def _metadata(src, tmp_path):
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC, src, "-o", out],
                   check=True, capture_output=True, text=True)
    text = open(out).read()
    doc = text.split(".amdgpu_metadata", 1)[1].split(".end_amdgpu_metadata", 1)[0]
    doc = "\n".join(line for line in doc.splitlines() if line.strip())  # drop the directive's indentation line
    return yaml.safe_load(doc)["amdhsa.kernels"]


def _world(name):
    """Template W of a kernel name (None for kernels without one; 0 for the rank-loop
    rank sum, which serves 9-16 ranks like the generic instances)."""
    if "reduce_loop_kernel" in name:
        return 0
    m = re.search(r"(row_kernel|splith_partial_kernel|scalar_kernel|reduce_kernel)ILi(\d+)E", name)
    return int(m.group(2)) if m else None


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="needs hipcc")
@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_kernel_code_objects(src, tmp_path):
    kernels = _metadata(src, tmp_path)
    assert kernels
    for k in kernels:
        name = k[".name"]
        assert k.get(".sgpr_spill_count", 0) == 0 and k.get(".vgpr_spill_count", 0) == 0, name
        assert k.get(".private_segment_fixed_size", 0) == 0, name
        hidden = [a[".value_kind"] for a in k.get(".args", []) if a[".value_kind"].startswith("hidden")]
        assert not hidden, (name, hidden)
        w = _world(name)
        generic = w in (0, 16)
        if not generic:
            assert k[".kernarg_segment_size"] <= MAX_FAST_ARGS, (name, k[".kernarg_segment_size"])
