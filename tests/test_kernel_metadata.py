"""Code-object properties of the gfx950 kernels, read from the metadata hipcc emits
for this repository's own sources (compiled here with the library's flags):

- no kernel spills registers or uses private (scratch) memory;
- no kernel needs the implicit-argument block (no blockDim / gridDim reads);
- every kernel specialised on W <= 8 (and the W-independent ones) takes at most
  112 bytes of arguments: on MI355X with ROCm 7 the host cost of a launch steps
  up by about 0.9 us beyond that, which matters for decode-sized calls;
- the flat-argument twins have their leading 14 argument dwords preloaded into
  scalar registers, the by-value kernels none.
"""
import os
import re
import subprocess

import pytest
import yaml

from residual_add_rmsnorm_arrms_amd import build as B

SOURCES = [os.path.join(B.CSRC, f) for f in ("arrms_kernels.hip", "arrms_reduce.hip")]
MAX_FAST_ARGS = 112


def _assembly(src, tmp_path):
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-I", B.INCLUDE, "-I", B.CSRC, src, "-o", out],
                   check=True, capture_output=True, text=True)
    return open(out).read()


def _metadata(src, tmp_path, text=None):
    text = text or _assembly(src, tmp_path)
    doc = text.split(".amdgpu_metadata", 1)[1].split(".end_amdgpu_metadata", 1)[0]
    doc = "\n".join(line for line in doc.splitlines() if line.strip())  # drop the directive's indentation line
    return yaml.safe_load(doc)["amdhsa.kernels"]


def _preload_lengths(text):
    """Kernel name -> dwords of arguments preloaded into scalar registers, from each
    kernel descriptor (.amdhsa_kernel ... .end_amdhsa_kernel)."""
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        n = re.search(r"\.amdhsa_user_sgpr_kernarg_preload_length (\d+)", m.group(2))
        out[m.group(1)] = int(n.group(1)) if n else 0
    return out


def _world(name):
    """Template W of a kernel name (None for kernels without one; 0 for the rank-loop
    rank sum, which serves 9-16 ranks like the generic instances)."""
    if "reduce_loop_kernel" in name:
        return 0
    m = re.search(r"(row_kernel|splith_partial_kernel|scalar_kernel|reduce_kernel)(?:_flat)?ILi(\d+)E", name)
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


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="needs hipcc")
@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(s) for s in SOURCES])
def test_flat_twins_preload_their_leading_arguments(src, tmp_path):
    """Every flat-argument twin (row, scalar, rank sum with W <= 8) has its leading 14
    argument dwords (sizes, residual, first partials) preloaded into scalar registers;
    the kernels taking one argument block by value have none (an aggregate cannot be)."""
    text = _assembly(src, tmp_path)
    lengths = _preload_lengths(text)
    names = [k[".name"] for k in _metadata(src, tmp_path, text)]
    flat = [n for n in names if "_flatILi" in n]
    # row: 27 (W, VPT) pairs x 2 store policies; scalar: 8 W x 3 load widths x 2; rank sum: 8 W x 6 (L, E)
    assert len(flat) == (102 if "kernels" in src else 48), len(flat)
    for n in names:
        want = 14 if n in flat else 0
        assert lengths.get(n) == want, (n, lengths.get(n))
        if n in flat:
            assert 1 <= _world(n) <= 8, n
