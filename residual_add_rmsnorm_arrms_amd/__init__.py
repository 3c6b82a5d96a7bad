"""Python binding of ``libarrms.so``: fused rank-partial sum + residual add + RMSNorm
on AMD Instinct MI355X (gfx950).

The C ABI (``include/arrms.h``) does all the work; every function here has the
C name and only marshals arguments (device pointers as Python ints, the stream
as a ``hipStream_t`` int).  ``FusedReduceResidualRMSNorm`` is a small operator
object over it that takes torch tensors: torch provides device memory and the
current stream, nothing else.  There is no CPU or eager fallback: without the
built library every call raises.

Operation (page "[TLERaw] Add NVSHMEM allreduce RMSNorm tutorial", FlagTree
PR #1122, section Summary; the operator/communicator wrapper of section
Implementation 5 is the model for the operator object):
    reduced = sum of W rank partials; residual_out = reduced + residual;
    norm_out = RMSNorm(residual_out, weight, eps), BF16 [T, H] rows.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

from .build import LIB as LIB_PATH

ARRMS_OK = 0
ARRMS_ERR_INVALID_ARG = 1
ARRMS_ERR_UNSUPPORTED = 2
ARRMS_ERR_HIP = 3
ARRMS_ERR_OOM = 4
ARRMS_ERR_SCRATCH = 5

ARRMS_VARIANT_AUTO = 0
ARRMS_VARIANT_ROW = 1
ARRMS_VARIANT_SPLITH = 2
ARRMS_VARIANT_SCALAR = 3
ARRMS_VARIANT_REDUCE = 4
ARRMS_VARIANT_REDUCE_SCALAR = 5

ARRMS_MAX_WORLD = 16
ARRMS_MAX_HIDDEN = 65536
ARRMS_ROW_MAX_HIDDEN = 16384
ARRMS_NOALLOC_SCRATCH_DOUBLES = 131072

# Every symbol include/arrms.h declares.
EXPORTS = ("arrms_create", "arrms_fused", "arrms_destroy", "arrms_status_string", "arrms_last_hip_error",
           "arrms_set_variant", "arrms_set_tuning", "arrms_plan", "arrms_query_plan", "arrms_reduce",
           "arrms_plan_reduce", "arrms_fused_noalloc")


class arrms_plan_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("variant", "grid", "block", "vec_per_thread", "threads_per_row",
                                            "rows_per_block", "chunks_per_row", "kernels", "blocks", "xcd_chunk",
                                            "elems_per_load", "residual_out_cached", "rank_loop",
                                            "kernarg_preload")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class arrms_tuning_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("vec_per_thread", "threads_per_row", "splith_block",
                                            "splith_max_tokens", "xcd_chunk", "rows_per_block", "scalar_elems",
                                            "residual_out_store", "kernarg_preload")]

    @classmethod
    def make(cls, vec_per_thread=0, threads_per_row=0, splith_block=0, splith_max_tokens=-1, xcd_chunk=-1,
             rows_per_block=0, scalar_elems=0, residual_out_store=0, kernarg_preload=0):
        return cls(vec_per_thread, threads_per_row, splith_block, splith_max_tokens, xcd_chunk, rows_per_block,
                   scalar_elems, residual_out_store, kernarg_preload)


class ArrmsError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, arrms_status_string(status), status))


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """The loaded ``libarrms.so``; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libarrms.so is not built (%s); run `python -m "
                                   "residual_add_rmsnorm_arrms_amd.build` or __graft_entry__.build()" % LIB_PATH)
            lib = ctypes.CDLL(LIB_PATH)
            vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            lib.arrms_create.argtypes = [ctypes.POINTER(vp), ci, ci, ci, ci]
            lib.arrms_fused.argtypes = [vp, ctypes.POINTER(vp), ci, ci, ci, vp, vp, cf, vp, vp, vp]
            lib.arrms_destroy.argtypes = [vp]
            lib.arrms_status_string.argtypes = [ci]
            lib.arrms_status_string.restype = ctypes.c_char_p
            lib.arrms_last_hip_error.argtypes = [vp]
            lib.arrms_set_variant.argtypes = [vp, ci]
            lib.arrms_set_tuning.argtypes = [vp, ctypes.POINTER(arrms_tuning_t)]
            lib.arrms_plan.argtypes = [ci, ci, ctypes.POINTER(arrms_tuning_t), ci, ci, ci, ctypes.POINTER(vp), ci,
                                       ci, ci, vp, vp, cf, vp, vp, ctypes.POINTER(arrms_plan_t)]
            lib.arrms_query_plan.argtypes = [vp, ctypes.POINTER(vp), ci, ci, ci, vp, vp, cf, vp, vp,
                                             ctypes.POINTER(arrms_plan_t)]
            lib.arrms_reduce.argtypes = [vp, ctypes.POINTER(vp), ci, ci, ci, vp, vp]
            lib.arrms_plan_reduce.argtypes = [ci, ctypes.POINTER(arrms_tuning_t), ci, ci, ci, ctypes.POINTER(vp), ci,
                                              ci, ci, vp, ctypes.POINTER(arrms_plan_t)]
            lib.arrms_fused_noalloc.argtypes = [ctypes.POINTER(vp), ci, ci, ci, vp, vp, cf, vp, vp, vp]
            _lib = lib
    return _lib


def _ptrs(partials: Optional[Sequence[int]]):
    if partials is None:
        return None
    return (ctypes.c_void_p * max(1, len(partials)))(*[p or None for p in partials])


# ---------------------------------------------------------------- raw C ABI
def arrms_create(device: int, max_world: int, max_tokens: int, max_hidden: int):
    """Returns (status, handle); handle is None on error."""
    h = ctypes.c_void_p()
    rc = load().arrms_create(ctypes.byref(h), device, max_world, max_tokens, max_hidden)
    return rc, (h.value if rc == ARRMS_OK else None)


def arrms_fused(h, partials: Optional[Sequence[int]], world: int, tokens: int, hidden: int, residual: int,
                weight: int, eps: float, residual_out: int, norm_out: int, stream: int = 0) -> int:
    return load().arrms_fused(h, _ptrs(partials), world, tokens, hidden, residual, weight, eps, residual_out,
                              norm_out, stream)


def arrms_fused_noalloc(partials: Optional[Sequence[int]], world: int, tokens: int, hidden: int, residual: int,
                        weight: int, eps: float, residual_out: int, norm_out: int, stream: int = 0) -> int:
    """arrms_fused without a handle or any allocation, on the current device (static scratch)."""
    return load().arrms_fused_noalloc(_ptrs(partials), world, tokens, hidden, residual, weight, eps, residual_out,
                                      norm_out, stream)


def arrms_destroy(h) -> int:
    return load().arrms_destroy(h)


def arrms_status_string(status: int) -> str:
    return load().arrms_status_string(status).decode()


def arrms_last_hip_error(h) -> int:
    return load().arrms_last_hip_error(h)


def arrms_set_variant(h, variant: int) -> int:
    return load().arrms_set_variant(h, variant)


def arrms_set_tuning(h, tuning: Optional[arrms_tuning_t]) -> int:
    return load().arrms_set_tuning(h, ctypes.byref(tuning) if tuning is not None else None)


def arrms_plan(cu_count: int, variant: int, tuning: Optional[arrms_tuning_t], max_world: int, max_tokens: int,
               max_hidden: int, partials: Optional[Sequence[int]], world: int, tokens: int, hidden: int,
               residual: int, weight: int, eps: float, residual_out: int, norm_out: int):
    """Host-only validation and planning. Returns (status, plan dict)."""
    p = arrms_plan_t()
    rc = load().arrms_plan(cu_count, variant, ctypes.byref(tuning) if tuning is not None else None, max_world,
                           max_tokens, max_hidden, _ptrs(partials), world, tokens, hidden, residual, weight, eps,
                           residual_out, norm_out, ctypes.byref(p))
    return rc, p.as_dict()


def arrms_query_plan(h, partials: Optional[Sequence[int]], world: int, tokens: int, hidden: int, residual: int,
                     weight: int, eps: float, residual_out: int, norm_out: int):
    """arrms_plan with a handle's settings. Returns (status, plan dict)."""
    p = arrms_plan_t()
    rc = load().arrms_query_plan(h, _ptrs(partials), world, tokens, hidden, residual, weight, eps, residual_out,
                                 norm_out, ctypes.byref(p))
    return rc, p.as_dict()


def arrms_reduce(h, partials: Optional[Sequence[int]], world: int, tokens: int, hidden: int, reduced: int,
                 stream: int = 0) -> int:
    return load().arrms_reduce(h, _ptrs(partials), world, tokens, hidden, reduced, stream)


def arrms_plan_reduce(cu_count: int, tuning: Optional[arrms_tuning_t], max_world: int, max_tokens: int,
                      max_hidden: int, partials: Optional[Sequence[int]], world: int, tokens: int, hidden: int,
                      reduced: int):
    """Host-only validation and planning of arrms_reduce. Returns (status, plan dict)."""
    p = arrms_plan_t()
    rc = load().arrms_plan_reduce(cu_count, ctypes.byref(tuning) if tuning is not None else None, max_world,
                                  max_tokens, max_hidden, _ptrs(partials), world, tokens, hidden, reduced,
                                  ctypes.byref(p))
    return rc, p.as_dict()


# ---------------------------------------------------------------- torch-facing operator
class BoundCall:
    """arrms_fused on buffers fixed at bind time (see FusedReduceResidualRMSNorm.bind)."""

    def __init__(self, owner, keep_alive, args, outputs):
        self._owner = owner
        self._keep = keep_alive
        self._args = args
        self._fn = load().arrms_fused
        self.outputs = outputs

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_fused")
        return self.outputs



class _TensorArgs:
    """Checks of the torch tensors of a call (BF16, contiguous, on `device`, shapes) and
    their device pointers; shared by the operator and fused_noalloc."""

    device: int

    def _check(self, t, name, shape=None):
        import torch
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("%s must be a bfloat16 GPU tensor" % name)
        if t.device.index != self.device:
            raise ValueError("%s is on cuda:%s, the call runs on cuda:%d" % (name, t.device.index, self.device))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))

    def _partial_ptrs(self, partials, T, H):
        """Device pointers of the W partials: a [W, T, H] tensor (checked once, pointers
        by stride, no per-rank views) or a sequence of W [T, H] tensors."""
        import torch
        if isinstance(partials, torch.Tensor) and partials.dim() == 3:
            if partials.is_contiguous():
                self._check(partials, "partials", (partials.shape[0], T, H))
                base, step = partials.data_ptr(), T * H * partials.element_size()
                return [base + r * step for r in range(partials.shape[0])]
            partials = partials.unbind(0)  # e.g. a token slice of a larger buffer: each rank's rows contiguous
        parts = list(partials)
        for i, p in enumerate(parts):
            self._check(p, "partials[%d]" % i, (T, H))
        return [p.data_ptr() for p in parts]

    def _args(self, partials, residual, weight, residual_out, norm_out):
        import torch
        if residual.dim() != 2:
            raise ValueError("residual must be [T, H]")
        T, H = residual.shape
        parts = self._partial_ptrs(partials, T, H)
        self._check(residual, "residual")
        self._check(weight, "weight", (H,))
        if residual_out is None:
            residual_out = torch.empty_like(residual)
        if norm_out is None:
            norm_out = torch.empty_like(residual)
        self._check(residual_out, "residual_out", (T, H))
        self._check(norm_out, "norm_out", (T, H))
        return parts, T, H, residual_out, norm_out


class FusedReduceResidualRMSNorm(_TensorArgs):
    """Reusable operator over one handle.  Tensors: BF16, on the handle's GPU.

    ``op(partials, residual, weight, eps, residual_out=None, norm_out=None)`` enqueues
    the fused call on torch's current stream and returns (residual_out, norm_out).
    ``partials`` is a [W, T, H] tensor or a sequence of W [T, H] tensors.

    One handle serves one call at a time (the split-H variant uses the handle's
    workspace): calls on the same stream are ordered by it, but calls on different
    streams must not overlap.  Use one operator per stream for concurrent streams.
    """

    def __init__(self, max_world: int, max_tokens: int, max_hidden: int, device: Optional[int] = None):
        import torch
        self.device = torch.cuda.current_device() if device is None else int(device)
        rc, h = arrms_create(self.device, max_world, max_tokens, max_hidden)
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_create")
        self.handle = h

    def set_variant(self, variant: int) -> None:
        rc = arrms_set_variant(self.handle, variant)
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_set_variant")

    def set_tuning(self, **kw) -> None:
        t = arrms_tuning_t.make(**kw) if kw else None
        rc = arrms_set_tuning(self.handle, t)
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_set_tuning")

    def plan(self, partials, residual, weight, eps, residual_out=None, norm_out=None) -> dict:
        parts, T, H, residual_out, norm_out = self._args(partials, residual, weight, residual_out, norm_out)
        rc, p = arrms_query_plan(self.handle, parts, len(parts), T, H, residual.data_ptr(),
                                 weight.data_ptr(), eps, residual_out.data_ptr(), norm_out.data_ptr())
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_query_plan")
        return p

    def __call__(self, partials, residual, weight, eps: float, residual_out=None, norm_out=None, stream=None):
        import torch
        parts, T, H, residual_out, norm_out = self._args(partials, residual, weight, residual_out, norm_out)
        s = (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream
        rc = arrms_fused(self.handle, parts, len(parts), T, H, residual.data_ptr(),
                         weight.data_ptr(), eps, residual_out.data_ptr(), norm_out.data_ptr(), s)
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_fused")
        return residual_out, norm_out

    def bind(self, partials, residual, weight, eps: float, residual_out=None, norm_out=None, stream=None):
        """A prepared call on fixed buffers: the tensors are checked and the C arguments
        marshalled once, and each call of the returned object only enqueues the kernel(s)
        (for serving loops on static buffers).  The tensors must stay alive and in place;
        the stream is fixed at bind time (torch's current stream by default)."""
        import torch
        ptrs, T, H, residual_out, norm_out = self._args(partials, residual, weight, residual_out, norm_out)
        s = (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream
        rc, _ = arrms_query_plan(self.handle, ptrs, len(ptrs), T, H, residual.data_ptr(), weight.data_ptr(), eps,
                                 residual_out.data_ptr(), norm_out.data_ptr())
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_fused")
        return BoundCall(self, (partials, residual, weight, residual_out, norm_out),
                         (ctypes.c_void_p(self.handle), _ptrs(ptrs), len(ptrs), T, H,
                          ctypes.c_void_p(residual.data_ptr()), ctypes.c_void_p(weight.data_ptr()),
                          ctypes.c_float(eps), ctypes.c_void_p(residual_out.data_ptr()),
                          ctypes.c_void_p(norm_out.data_ptr()), ctypes.c_void_p(s)),
                         (residual_out, norm_out))

    def reduce(self, partials, reduced=None, stream=None):
        """reduced = BF16 rank sum of the partials ([W, T, H] or W x [T, H]); returns reduced."""
        import torch
        first = partials[0]
        T, H = first.shape
        ptrs = self._partial_ptrs(partials, T, H)
        if reduced is None:
            reduced = torch.empty((T, H), dtype=first.dtype, device=first.device)
        self._check(reduced, "reduced", (T, H))
        s = (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream
        rc = arrms_reduce(self.handle, ptrs, len(ptrs), T, H, reduced.data_ptr(), s)
        if rc != ARRMS_OK:
            raise ArrmsError(rc, "arrms_reduce")
        return reduced

    def close(self) -> None:
        """Destroy the handle (synchronise the stream of the last call first)."""
        if getattr(self, "handle", None) is not None:
            arrms_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def fused_noalloc(partials, residual, weight, eps: float, residual_out, norm_out, stream=None):
    """arrms_fused_noalloc on torch tensors: the fused call on the current device with no
    handle and no allocation of any kind (for code under graph capture or in serving
    loops).  Both outputs must be given; tensors as for FusedReduceResidualRMSNorm.
    The first call on a device looks up its static scratch and should be made outside
    graph capture.  Returns (residual_out, norm_out)."""
    import torch
    if residual_out is None or norm_out is None:
        raise ValueError("fused_noalloc allocates nothing: pass residual_out and norm_out")
    args = _TensorArgs()
    args.device = torch.cuda.current_device()
    parts, T, H, residual_out, norm_out = args._args(partials, residual, weight, residual_out, norm_out)
    s = (stream if stream is not None else torch.cuda.current_stream(args.device)).cuda_stream
    rc = arrms_fused_noalloc(parts, len(parts), T, H, residual.data_ptr(), weight.data_ptr(), eps,
                             residual_out.data_ptr(), norm_out.data_ptr(), s)
    if rc != ARRMS_OK:
        raise ArrmsError(rc, "arrms_fused_noalloc")
    return residual_out, norm_out
