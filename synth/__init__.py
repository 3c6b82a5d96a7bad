"""Seeded synthetic inputs for the fused rank-sum + residual add + RMSNorm operator.

This module only draws numbers (see ``synth.c``); it holds no step of the
operator's arithmetic.  The CPU oracle and the GPU library are both fed the
exact bytes it returns, so a parity test compares the two on identical inputs.

Tensors come back as CPU ``torch.bfloat16`` tensors; the binary32 samples are
rounded to bfloat16 by torch's own conversion (round to nearest, ties to even).

Workloads follow the page "[TLERaw] Add NVSHMEM allreduce RMSNorm tutorial"
(FlagTree PR #1122): section Correctness validates world size 4, hidden size
2048, BF16, tokens 1 ... 4096.  Value distributions (N(0,1) partials and
residual, U(0.5, 1.5) weight, eps 1e-6) are this package's synthetic choice,
since the page does not give them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

# Stream tags: one independent stream per tensor and per rank.
TAG_RESIDUAL = 1000
TAG_WEIGHT = 1001
TAG_OUTLIER_BASE = 2000


def build(force: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP for speed; bytes do not depend on threads)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_uint64, ctypes.c_double, ctypes.c_double]
            lib.synth_normal.restype = None
            lib.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double, ctypes.c_double,
                                          ctypes.c_int64, ctypes.c_void_p]
            lib.synth_uniform.restype = None
            _lib = lib
    return _lib


def normal_f32(seed: int, tag: int, sigma: float, n: int, outlier_p: float = 0.0,
               outlier_scale: float = 100.0, outlier_tag: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal(seed, tag, sigma, n, out.ctypes.data, outlier_tag, outlier_p, outlier_scale)
    return out


def uniform_f32(seed: int, tag: int, lo: float, hi: float, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_uniform(seed, tag, lo, hi, n, out.ctypes.data)
    return out


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """binary32 -> bfloat16 through torch's conversion (round to nearest, ties to even)."""
    return torch.from_numpy(a).to(torch.bfloat16)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value distributions and eps."""
    name: str
    world: int
    tokens: int
    hidden: int
    x_sigma: float = 1.0
    residual_sigma: float = 1.0
    weight_lo: float = 0.5
    weight_hi: float = 1.5
    eps: float = 1e-6
    outlier_p: float = 0.0
    outlier_scale: float = 100.0
    seed: int = 0

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes one call must move: read W partials + residual, write two outputs, read weight once."""
        return 2 * self.tokens * self.hidden * (self.world + 3) + 2 * self.hidden

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The named workloads.  Shapes: tiny W=2 T=4 H=128; decode W=4 H=2048 T in {1,16,128};
# prefill W=4 H=2048 T=4096 with partials ~N(0, 0.5^2); large hidden W=8 H=8192 T=8192, eps 1e-5;
# ragged + outliers W=8 H=5120 T=16383, 1% of partial entries scaled by 100; odd rows: the
# prefill shape with H=2047 (rows the 16-byte kernels cannot take, for the scalar kernel's profile).
WORKLOADS = {
    "tiny": Workload("tiny", 2, 4, 128),
    "decode_t1": Workload("decode_t1", 4, 1, 2048),
    "decode_t16": Workload("decode_t16", 4, 16, 2048),
    "decode_t128": Workload("decode_t128", 4, 128, 2048),
    "prefill": Workload("prefill", 4, 4096, 2048, x_sigma=0.5),
    "large_hidden": Workload("large_hidden", 8, 8192, 8192, eps=1e-5),
    "ragged_outliers": Workload("ragged_outliers", 8, 16383, 5120, outlier_p=0.01),
    "odd_rows": Workload("odd_rows", 4, 4096, 2047, x_sigma=0.5),
}


def make_inputs(wl: Workload):
    """Return (x [W,T,H], residual [T,H], weight [H]) as CPU bfloat16 tensors for workload ``wl``."""
    W, T, H = wl.world, wl.tokens, wl.hidden
    x = torch.empty((W, T, H), dtype=torch.bfloat16)
    for r in range(W):
        a = normal_f32(wl.seed, r, wl.x_sigma, T * H, wl.outlier_p, wl.outlier_scale, TAG_OUTLIER_BASE + r)
        x[r].copy_(to_bf16(a).view(T, H))
        del a
    residual = to_bf16(normal_f32(wl.seed, TAG_RESIDUAL, wl.residual_sigma, T * H)).view(T, H)
    weight = to_bf16(uniform_f32(wl.seed, TAG_WEIGHT, wl.weight_lo, wl.weight_hi, H))
    return x, residual, weight


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 numpy view of a CPU bfloat16 tensor's bit patterns (no copy when contiguous)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    """CPU bfloat16 tensor with the bit patterns of uint16 array ``a``."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
