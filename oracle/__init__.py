"""CPU oracle for the fused rank-sum + residual add + RMSNorm operator.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, nothing else.  The GPU library never
imports or calls it and has no fallback to it.

The arithmetic lives in ``arrms_oracle.c`` (plain scalar C, one IEEE operation per
step, no FMA contraction); it follows the contract of the page "[TLERaw] Add
NVSHMEM allreduce RMSNorm tutorial" (FlagTree PR #1122), section Summary and
section Implementation 3, with the readings listed at the top of that file.
This module only marshals numpy arrays into it.

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, invariants, library routines and hand-derived fixtures; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "arrms_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# gcc flags: plain IEEE scalar arithmetic (x86-64 SSE2), no fast-math, no contraction.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
          "-fno-unsafe-math-optimizations"]


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``liboracle.so`` (or ``out``) from ``arrms_oracle.c`` (or ``src``) with gcc."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class Oracle:
    """The oracle library at ``lib_path`` (the default is this directory's ``liboracle.so``)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        vp = ctypes.c_void_p
        lib.oracle_fused_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                          ctypes.c_float, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int]
        lib.oracle_fused_rows.restype = ctypes.c_int
        lib.oracle_round_bf16.argtypes = [ctypes.c_float]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_bf16_bits.argtypes = [ctypes.c_uint32]
        lib.oracle_round_bf16_bits.restype = ctypes.c_uint16
        lib.oracle_widen_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_widen_bf16.restype = ctypes.c_float
        self.lib = lib
        self.path = lib_path

    def round_bf16(self, f: float) -> int:
        """BF16 bit pattern of binary32 ``f`` rounded to nearest, ties to even."""
        return int(self.lib.oracle_round_bf16(ctypes.c_float(f)))

    def round_bf16_bits(self, u: int) -> int:
        """BF16 bit pattern of the binary32 with bit pattern ``u``, rounded to nearest even."""
        return int(self.lib.oracle_round_bf16_bits(ctypes.c_uint32(u)))

    def widen_bf16(self, b: int) -> float:
        """binary32 value of BF16 bit pattern ``b`` (exact)."""
        return float(self.lib.oracle_widen_bf16(ctypes.c_uint16(b)))

    def fused(self, x, residual, weight, eps: float, rows: tuple[int, int] | None = None, threads: int = 1):
        """Run the operator on BF16 bit patterns.

        x        : uint16 [W, T, H] (or a sequence of W uint16 [T, H] arrays)
        residual : uint16 [T, H]
        weight   : uint16 [H]
        rows     : optional (begin, end) row range; other rows of the outputs stay 0
        threads  : split the row range into this many contiguous pieces, one host thread
                   each (rows are independent, so the result does not depend on it)

        Returns a dict of uint16 arrays ``reduced``, ``residual_out``, ``norm_out``
        ([T, H] each) and the binary32 per-row ``inv_rms`` [T].
        """
        xs = [_u16(p) for p in x]
        residual = _u16(residual)
        weight = _u16(weight)
        W = len(xs)
        T, H = residual.shape
        for p in xs:
            if p.shape != (T, H):
                raise ValueError("partial shape %s != residual shape %s" % (p.shape, (T, H)))
        if weight.shape != (H,):
            raise ValueError("weight shape %s != (%d,)" % (weight.shape, H))
        b, e = rows if rows is not None else (0, T)
        ptrs = (ctypes.c_void_p * W)(*[p.ctypes.data for p in xs])
        out = {k: np.zeros((T, H), dtype=np.uint16) for k in ("reduced", "residual_out", "norm_out")}
        out["inv_rms"] = np.zeros(T, dtype=np.float32)
        ranges = [(b, e)]
        if threads > 1 and e - b > 1:
            n = min(threads, e - b)
            ranges = [(b + (e - b) * i // n, b + (e - b) * (i + 1) // n) for i in range(n)]
        status = [0] * len(ranges)

        def run(i):
            rb, re_ = ranges[i]
            status[i] = self.lib.oracle_fused_rows(
                W, T, H, ptrs, residual.ctypes.data, weight.ctypes.data, ctypes.c_float(eps),
                out["reduced"].ctypes.data, out["residual_out"].ctypes.data, out["norm_out"].ctypes.data,
                out["inv_rms"].ctypes.data, rb, re_)

        if len(ranges) == 1:
            run(0)
        else:
            # rows are independent; ctypes releases the GIL during each foreign call
            workers = [threading.Thread(target=run, args=(i,)) for i in range(len(ranges))]
            for t in workers:
                t.start()
            for t in workers:
                t.join()
        if any(status):
            raise ValueError("oracle rejected its arguments")
        return out


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are BF16 bit patterns (uint16), got %s" % a.dtype)
    return np.ascontiguousarray(a)


def default() -> Oracle:
    """The oracle built from ``arrms_oracle.c`` (compiled on first use if missing or stale)."""
    global _lib
    with _lock:
        if _lib is None:
            _lib = Oracle(build())
    return _lib


def round_bf16(f: float) -> int:
    return default().round_bf16(f)


def widen_bf16(b: int) -> float:
    return default().widen_bf16(b)


def fused(x, residual, weight, eps: float, rows: tuple[int, int] | None = None, threads: int = 1):
    return default().fused(x, residual, weight, eps, rows, threads)
