"""Python binding of the HIP library ``libargreduce.so`` (argument marshalling only).

ctypes loads the library and serves every entry point; the three reduction calls go
through a small CPython fast-call module (``_argreduce_fast``, built beside the library)
when it is present, because a ctypes call with nine converted arguments costs about as
much host time as the GPU spends on a small reduction.

The functions carry the names of the C ABI in include/argreduce.h and take the same
arguments (device pointers as Python ints). ``argmax`` / ``argmin`` are conveniences for
torch tensors: torch supplies the device memory (output and scratch) and the current
HIP stream; every step of the reduction runs in the library's kernels. There is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libargreduce.so")

# enums of include/argreduce.h
F32, F16, BF16, F64, I32, I64 = 0, 1, 2, 3, 4, 5
MAX, MIN, MAX_LAST, MIN_LAST = 0, 1, 2, 3
PATH_AUTO, PATH_SUBWAVE, PATH_BLOCK, PATH_SPLIT, PATH_AXIS, PATH_SCAN, PATH_WIDE = -1, 0, 1, 2, 3, 4, 5
PATH_THREAD = 6  # forced only: one lane per row (the serial "before" kernel)
OK = 0
ERRORS = {
    -1: "ARGREDUCE_ERR_INVALID_ARG",
    -2: "ARGREDUCE_ERR_UNSUPPORTED_DTYPE",
    -3: "ARGREDUCE_ERR_TOO_WIDE",
    -4: "ARGREDUCE_ERR_SCRATCH_TOO_SMALL",
    -5: "ARGREDUCE_ERR_HIP",
    -6: "ARGREDUCE_ERR_NO_DEVICE",
}
DTYPE_NAMES = {"f32": F32, "f16": F16, "bf16": BF16, "f64": F64, "i32": I32, "i64": I64}
OP_NAMES = {"max": MAX, "min": MIN, "max_last": MAX_LAST, "min_last": MIN_LAST}
SIZE_MAX = ctypes.c_size_t(-1).value

# Exported names of include/argreduce.h (checked by the CPU test suite).
EXPORTS = ("argreduce_scratch_bytes", "argreduce_lastaxis", "argreduce_plan",
           "argreduce_debug_set_capacity", "argreduce_debug_force_path", "argreduce_debug_force_split",
           "argreduce_debug_launch_empty", "argreduce_debug_set_kernel_events",
           "argreduce_axis_scratch_bytes", "argreduce_axis", "argreduce_axis_plan",
           "argreduce_scan_scratch_bytes", "argreduce_scan_lastaxis", "argreduce_scan_plan",
           "argreduce_debug_set_window", "argreduce_debug_launch_store",
           "argreduce_debug_set_spin_limit", "argreduce_debug_launch_read",
           "argreduce_wait_timeouts", "argreduce_lastaxis_noalloc")


class ArgreduceError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({code})")
        self.code = code


class argreduce_plan_t(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("lanes_per_row", ctypes.c_int32),
                ("blocks_per_row", ctypes.c_int32), ("block_threads", ctypes.c_int32),
                ("grid_blocks", ctypes.c_int64), ("grid_rows", ctypes.c_int64),
                ("unroll", ctypes.c_int32), ("outputs_per_block", ctypes.c_int32),
                ("device_threads", ctypes.c_int64), ("scratch_bytes", ctypes.c_size_t),
                ("load_bytes", ctypes.c_int32), ("dispatches", ctypes.c_int32),
                ("window", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m argmin_reduction_wide_amd.build` (no fallback exists)")
                # torch ships its own HIP runtime; importing it first makes the library
                # bind to that one (same soname), so torch's streams and allocations
                # belong to the runtime that launches our kernels.
                try:
                    import torch  # noqa: F401
                except ImportError:
                    pass
                h = ctypes.CDLL(LIB_PATH)
                i64, sz, vp, c_int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
                h.argreduce_scratch_bytes.argtypes = [i64, i64, c_int]
                h.argreduce_scratch_bytes.restype = sz
                h.argreduce_lastaxis.argtypes = [vp, c_int, i64, i64, c_int, vp, vp, sz, vp]
                h.argreduce_lastaxis.restype = c_int
                h.argreduce_plan.argtypes = [i64, i64, c_int, ctypes.POINTER(argreduce_plan_t)]
                h.argreduce_plan.restype = c_int
                h.argreduce_debug_set_capacity.argtypes = [i64]
                h.argreduce_debug_set_capacity.restype = c_int
                h.argreduce_debug_force_path.argtypes = [c_int]
                h.argreduce_debug_force_path.restype = c_int
                h.argreduce_debug_force_split.argtypes = [i64, c_int]
                h.argreduce_debug_force_split.restype = c_int
                h.argreduce_axis_scratch_bytes.argtypes = [i64, i64, i64, c_int]
                h.argreduce_axis_scratch_bytes.restype = sz
                h.argreduce_axis.argtypes = [vp, c_int, i64, i64, i64, c_int, vp, vp, sz, vp]
                h.argreduce_axis.restype = c_int
                h.argreduce_axis_plan.argtypes = [i64, i64, i64, c_int,
                                                  ctypes.POINTER(argreduce_plan_t)]
                h.argreduce_axis_plan.restype = c_int
                h.argreduce_scan_scratch_bytes.argtypes = [i64, i64, c_int]
                h.argreduce_scan_scratch_bytes.restype = sz
                h.argreduce_scan_lastaxis.argtypes = [vp, c_int, i64, i64, c_int, vp, vp, vp, sz, vp]
                h.argreduce_scan_lastaxis.restype = c_int
                h.argreduce_scan_plan.argtypes = [i64, i64, c_int, ctypes.POINTER(argreduce_plan_t)]
                h.argreduce_scan_plan.restype = c_int
                h.argreduce_debug_launch_store.argtypes = [vp, vp]
                h.argreduce_debug_launch_store.restype = c_int
                h.argreduce_debug_launch_read.argtypes = [vp, sz, vp, i64, vp]
                h.argreduce_debug_launch_read.restype = c_int
                h.argreduce_debug_set_spin_limit.argtypes = [ctypes.c_uint32]
                h.argreduce_debug_set_spin_limit.restype = c_int
                h.argreduce_lastaxis_noalloc.argtypes = [vp, c_int, i64, i64, c_int, vp, vp]
                h.argreduce_lastaxis_noalloc.restype = c_int
                h.argreduce_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
                h.argreduce_wait_timeouts.restype = c_int
                h.argreduce_debug_set_window.argtypes = [i64]
                h.argreduce_debug_set_window.restype = c_int
                h.argreduce_debug_launch_empty.argtypes = [vp]
                h.argreduce_debug_launch_empty.restype = c_int
                h.argreduce_debug_set_kernel_events.argtypes = [vp, vp]
                h.argreduce_debug_set_kernel_events.restype = c_int
                _bind_fast(h)
                _lib = h
    return _lib


_fast = None


def _bind_fast(h: ctypes.CDLL) -> None:
    """Hand the library's reduction entry points (and launch-floor hooks) to the CPython
    fast-call module, when it has been built: it marshals the same arguments with far less
    host time per call than ctypes. Without it the ctypes functions serve."""
    global _fast
    try:
        from . import _argreduce_fast as m
    except ImportError:
        return
    addr = lambda f: ctypes.cast(f, ctypes.c_void_p).value
    m.bind(addr(h.argreduce_lastaxis), addr(h.argreduce_axis), addr(h.argreduce_scan_lastaxis),
           addr(h.argreduce_debug_launch_empty), addr(h.argreduce_debug_launch_store),
           addr(h.argreduce_debug_launch_read))
    _fast = m


def fast():
    """The fast-call module bound to the loaded library, or None when it is not built. Its
    functions take the C ABI's arguments as ints (enum codes, not names)."""
    lib()
    return _fast


def entry_point(name: str):
    """A reduction entry point: the fast-call one when built, else the ctypes one."""
    h = lib()
    return getattr(_fast, name) if _fast is not None else getattr(h, name)


def _dtype_code(dtype) -> int:
    return DTYPE_NAMES[dtype] if isinstance(dtype, str) else int(dtype)


def _op_code(op) -> int:
    return OP_NAMES[op] if isinstance(op, str) else int(op)


# ---------------------------------------------------------------------------------------
# C ABI, one Python function per exported symbol


def argreduce_scratch_bytes(rows: int, cols: int, dtype) -> int:
    """Scratch bytes for this shape on the current device; SIZE_MAX on invalid input."""
    return lib().argreduce_scratch_bytes(rows, cols, _dtype_code(dtype))


def argreduce_lastaxis(x_ptr: int, dtype, rows: int, cols: int, op, out_ptr: int,
                       scratch_ptr: int, scratch_bytes: int, stream: int) -> int:
    """Enqueue the reduction; returns the library's status code (0 = success)."""
    return entry_point("argreduce_lastaxis")(x_ptr, _dtype_code(dtype), rows, cols, _op_code(op),
                                        out_ptr, scratch_ptr, scratch_bytes, stream)


# Bytes of the library-held scratch of argreduce_lastaxis_noalloc (include/argreduce.h).
NOALLOC_SCRATCH_BYTES = 128 * 1024


def argreduce_lastaxis_noalloc(x_ptr: int, dtype, rows: int, cols: int, op, out_ptr: int,
                               stream: int) -> int:
    """argreduce_lastaxis with the library-held scratch (no scratch argument, nothing
    allocated); returns the library's status code."""
    return lib().argreduce_lastaxis_noalloc(x_ptr, _dtype_code(dtype), rows, cols, _op_code(op),
                                            out_ptr, stream)


def argreduce_plan(rows: int, cols: int, dtype) -> dict:
    p = argreduce_plan_t()
    rc = lib().argreduce_plan(rows, cols, _dtype_code(dtype), ctypes.byref(p))
    if rc != OK:
        raise ArgreduceError(rc, "argreduce_plan")
    return p.as_dict()


def argreduce_axis_scratch_bytes(outer: int, length: int, inner: int, dtype) -> int:
    return lib().argreduce_axis_scratch_bytes(outer, length, inner, _dtype_code(dtype))


def argreduce_axis(x_ptr: int, dtype, outer: int, length: int, inner: int, op, out_ptr: int,
                   scratch_ptr: int, scratch_bytes: int, stream: int) -> int:
    return entry_point("argreduce_axis")(x_ptr, _dtype_code(dtype), outer, length, inner,
                                    _op_code(op), out_ptr, scratch_ptr, scratch_bytes, stream)


def argreduce_axis_plan(outer: int, length: int, inner: int, dtype) -> dict:
    p = argreduce_plan_t()
    rc = lib().argreduce_axis_plan(outer, length, inner, _dtype_code(dtype), ctypes.byref(p))
    if rc != OK:
        raise ArgreduceError(rc, "argreduce_axis_plan")
    return p.as_dict()


def argreduce_scan_scratch_bytes(rows: int, cols: int, dtype) -> int:
    return lib().argreduce_scan_scratch_bytes(rows, cols, _dtype_code(dtype))


def argreduce_scan_lastaxis(x_ptr: int, dtype, rows: int, cols: int, op, values_ptr: int,
                            idx_ptr: int, scratch_ptr: int, scratch_bytes: int, stream: int) -> int:
    return entry_point("argreduce_scan_lastaxis")(x_ptr, _dtype_code(dtype), rows, cols,
                                             _op_code(op), values_ptr, idx_ptr, scratch_ptr,
                                             scratch_bytes, stream)


def argreduce_scan_plan(rows: int, cols: int, dtype) -> dict:
    p = argreduce_plan_t()
    rc = lib().argreduce_scan_plan(rows, cols, _dtype_code(dtype), ctypes.byref(p))
    if rc != OK:
        raise ArgreduceError(rc, "argreduce_scan_plan")
    return p.as_dict()


def argreduce_debug_set_capacity(threads: int) -> int:
    return lib().argreduce_debug_set_capacity(threads)


def argreduce_debug_launch_store(out_ptr: int, stream: int) -> int:
    return entry_point("argreduce_debug_launch_store")(out_ptr, stream)


def argreduce_debug_launch_read(x_ptr: int, nbytes: int, out_ptr: int, grid: int,
                                stream: int) -> int:
    return entry_point("argreduce_debug_launch_read")(x_ptr, nbytes, out_ptr, grid, stream)


def argreduce_debug_set_spin_limit(polls: int) -> int:
    return lib().argreduce_debug_set_spin_limit(polls)


def argreduce_wait_timeouts() -> int:
    """Bounded waits that gave up on the current device since the library was loaded
    (synchronous read of a device counter); raises ArgreduceError on failure."""
    c = ctypes.c_uint64(0)
    rc = lib().argreduce_wait_timeouts(ctypes.byref(c))
    if rc != 0:
        raise ArgreduceError(rc, "argreduce_wait_timeouts")
    return c.value


def argreduce_debug_set_window(elements: int) -> int:
    return lib().argreduce_debug_set_window(elements)


def argreduce_debug_force_path(path: int) -> int:
    return lib().argreduce_debug_force_path(path)


def argreduce_debug_force_split(blocks_per_row: int, unroll: int = 1) -> int:
    """Force the split geometry of last-axis plans (0 restores the automatic plans)."""
    return lib().argreduce_debug_force_split(blocks_per_row, unroll)


def argreduce_debug_launch_empty(stream: int) -> int:
    return entry_point("argreduce_debug_launch_empty")(stream)


def argreduce_debug_set_kernel_events(start: int, stop: int) -> int:
    return lib().argreduce_debug_set_kernel_events(start, stop)


# ---------------------------------------------------------------------------------------
# torch conveniences

_TORCH_DTYPES = None


def _torch_dtype_code(t) -> int:
    global _TORCH_DTYPES
    import torch

    if _TORCH_DTYPES is None:
        _TORCH_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16,
                         torch.float64: F64, torch.int32: I32, torch.int64: I64}
    try:
        return _TORCH_DTYPES[t.dtype]
    except KeyError:
        raise ArgreduceError(-2, f"argreduce on {t.dtype}") from None


def _check_buffer(b, name: str, device, dtype=None, numel=None) -> None:
    """A caller-supplied output or scratch tensor: on the input's device and contiguous,
    and, for an output, int64 with one element per result. The kernels write through its
    address with no bounds of their own, so a mismatch is refused before anything runs."""
    if not b.is_cuda or b.device != device:
        raise ValueError(f"{name} must be on {device}; got {b.device}")
    if not b.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and b.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}; got {b.dtype}")
    if numel is not None and b.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements; got {b.numel()}")


def _reduce(t, op: int, out=None, scratch=None, dim: int = -1):
    import math

    import torch

    if not t.is_cuda:
        raise ValueError("argreduce runs on the GPU only; got a CPU tensor")
    if t.dim() == 0:
        raise ValueError("argreduce needs at least one dimension")
    if not t.is_contiguous():
        raise ValueError("argreduce needs a contiguous tensor")
    dim = dim % t.dim()
    dtype = _torch_dtype_code(t)
    outer = math.prod(t.shape[:dim])
    length = t.shape[dim]
    inner = math.prod(t.shape[dim + 1:])
    if out is None:
        out = torch.empty(t.shape[:dim] + t.shape[dim + 1:], dtype=torch.int64, device=t.device)
    else:
        _check_buffer(out, "out", t.device, torch.int64, outer * inner)
    need = argreduce_axis_scratch_bytes(outer, length, inner, dtype)
    if need == SIZE_MAX:
        raise ArgreduceError(-1, f"argreduce_axis_scratch_bytes({outer}, {length}, {inner})")
    if scratch is not None:
        _check_buffer(scratch, "scratch", t.device)
    if need and (scratch is None or scratch.numel() * scratch.element_size() < need):
        scratch = torch.empty(need, dtype=torch.uint8, device=t.device)
    sptr = scratch.data_ptr() if (need and scratch is not None) else 0
    sbytes = scratch.numel() * scratch.element_size() if (need and scratch is not None) else 0
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = argreduce_axis(t.data_ptr(), dtype, outer, length, inner, op, out.data_ptr(), sptr,
                        sbytes, stream)
    if rc != OK:
        raise ArgreduceError(rc, f"argreduce_axis(outer={outer}, len={length}, inner={inner})")
    return out


def argmax(t, dim: int = -1, out=None, scratch=None, select_last_index: bool = False,
           keepdim: bool = False):
    """Index of the maximum along `dim` (first occurrence, or the last with
    select_last_index; NaN is never selected, a leading NaN gives 0). With keepdim the
    result keeps `dim` with size 1 (a view of `out`)."""
    r = _reduce(t, MAX_LAST if select_last_index else MAX, out, scratch, dim)
    return r.unsqueeze(dim % t.dim()) if keepdim else r


def argmin(t, dim: int = -1, out=None, scratch=None, select_last_index: bool = False,
           keepdim: bool = False):
    """Index of the minimum along `dim` (first occurrence, or the last with
    select_last_index; NaN is never selected, a leading NaN gives 0). With keepdim the
    result keeps `dim` with size 1 (a view of `out`)."""
    r = _reduce(t, MIN_LAST if select_last_index else MIN, out, scratch, dim)
    return r.unsqueeze(dim % t.dim()) if keepdim else r


def _scan(t, op: int, dim: int, scratch=None):
    import torch

    if not t.is_cuda:
        raise ValueError("the scan runs on the GPU only; got a CPU tensor")
    if t.dim() == 0:
        raise ValueError("the scan needs at least one dimension")
    if not t.is_contiguous():
        raise ValueError("the scan needs a contiguous tensor")
    if dim % t.dim() != t.dim() - 1:
        raise ValueError("the scan runs along the last dimension only")
    dtype = _torch_dtype_code(t)
    cols = t.shape[-1]
    rows = t.numel() // cols if cols else 0
    values = torch.empty_like(t)
    indices = torch.empty(t.shape, dtype=torch.int64, device=t.device)
    need = argreduce_scan_scratch_bytes(rows, cols, dtype)
    if need == SIZE_MAX:
        raise ArgreduceError(-1, f"argreduce_scan_scratch_bytes({rows}, {cols})")
    if scratch is not None:
        _check_buffer(scratch, "scratch", t.device)
    if need and (scratch is None or scratch.numel() * scratch.element_size() < need):
        scratch = torch.empty(need, dtype=torch.uint8, device=t.device)
    sptr = scratch.data_ptr() if need else 0
    sbytes = scratch.numel() * scratch.element_size() if need else 0
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = argreduce_scan_lastaxis(t.data_ptr(), dtype, rows, cols, op, values.data_ptr(),
                                 indices.data_ptr(), sptr, sbytes, stream)
    if rc != OK:
        raise ArgreduceError(rc, f"argreduce_scan_lastaxis(rows={rows}, cols={cols})")
    return values, indices


def cummax(t, dim: int = -1, scratch=None):
    """(values, indices) of the running maximum along the last dimension: at every position
    the ArgMax of the prefix (ties keep the earlier index, NaN never taken after position 0,
    a leading NaN holds) and the element there."""
    return _scan(t, MAX, dim, scratch)


def cummin(t, dim: int = -1, scratch=None):
    """(values, indices) of the running minimum along the last dimension (as cummax)."""
    return _scan(t, MIN, dim, scratch)
