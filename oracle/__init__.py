"""CPU oracle for the last-axis ArgMax / ArgMin reduction.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path (the
HIP library and its Python binding) never imports, loads or calls anything here, and
this package imports nothing from the product path.

The arithmetic lives in ``argreduce_oracle.c``: the sequential strict-compare scan seeded
at element 0 that the ONNX Runtime pages use as the definition of the result
("[CUDA] Parallelize ArgMax/ArgMin over wide last axes", Description / Semantics;
"[CUDA] Parallelize ArgMax/ArgMin over the reduction axis", Semantics), and the same scan
reported at every position for cummax / cummin (the PaddlePaddle issue on the cummax /
cummin kernel, fix proposals: an ArgMax-style (value, index) operator, ties to the
earlier index). This module only
compiles it with gcc and marshals numpy arrays into it.

Element formats are given as strings: ``"f32"`` (numpy float32), ``"f16"`` (numpy
float16), ``"bf16"`` (numpy uint16 holding bfloat16 bit patterns), ``"f64"`` (numpy
float64) and, for the cumulative scan only, ``"i32"`` / ``"i64"`` (numpy int32 / int64). Ops are ``"max"`` (ArgMax), ``"min"`` (ArgMin), and ``"max_last"`` /
``"min_last"`` (ties to the last index, ONNX's select_last_index = 1: the same scan with
a non-strict comparison).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "argreduce_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_argreduce.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3, "i32": 4, "i64": 5}
OP_CODE = {"max": 0, "min": 1, "max_last": 2, "min_last": 3}
NUMPY_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "f64": np.float64,
                 "i32": np.int32, "i64": np.int64}

# -O2, IEEE semantics: no -ffast-math, no -ffinite-math-only, no flush-to-zero.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = _SRC, out: str = _LIB, extra_flags: list[str] | None = None) -> str:
    """Compile the oracle (or a variant of its source) into a shared library."""
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes handle on one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        f = lib.oracle_argreduce_lastaxis
        f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_void_p]
        f.restype = ctypes.c_int
        a = lib.oracle_argreduce_axis
        a.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        a.restype = ctypes.c_int
        self._a = a
        c = lib.oracle_cumulative
        c.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_void_p]
        c.restype = ctypes.c_int
        self._c = c
        d = lib.oracle_widen
        d.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
        d.restype = ctypes.c_int
        self._lib, self._f, self._d = lib, f, d

    def argreduce_lastaxis(self, x: np.ndarray, dtype: str, op: str) -> np.ndarray:
        """int64 index per row of the 2-D array ``x`` (rows, cols)."""
        x = _as_storage(x, dtype)
        rows, cols = x.shape
        out = np.empty(rows, dtype=np.int64)
        rc = self._f(x.ctypes.data, DTYPE_CODE[dtype], rows, cols, OP_CODE[op], out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected rows={rows} cols={cols} dtype={dtype} op={op}")
        return out

    def argreduce_axis(self, x: np.ndarray, dtype: str, op: str) -> np.ndarray:
        """int64 index over the middle axis of the 3-D array ``x`` (outer, len, inner);
        result shape (outer, inner)."""
        want = NUMPY_STORAGE[dtype]
        if x.dtype != want or x.ndim != 3:
            raise TypeError(f"{dtype} data must be a 3-D {np.dtype(want)} array")
        x = np.ascontiguousarray(x)
        outer, length, inner = x.shape
        out = np.empty((outer, inner), dtype=np.int64)
        rc = self._a(x.ctypes.data, DTYPE_CODE[dtype], outer, length, inner, OP_CODE[op],
                     out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected shape {x.shape} dtype={dtype} op={op}")
        return out

    def cumulative(self, x: np.ndarray, dtype: str, op: str) -> tuple[np.ndarray, np.ndarray]:
        """Running extremum of every row prefix of the 2-D array ``x``: (values, indices),
        values in ``x``'s storage format, indices int64, both of ``x``'s shape. ``op`` is
        ``"max"`` (cummax) or ``"min"`` (cummin)."""
        x = _as_storage(x, dtype)
        rows, cols = x.shape
        vals = np.empty_like(x)
        idx = np.empty((rows, cols), dtype=np.int64)
        rc = self._c(x.ctypes.data, DTYPE_CODE[dtype], rows, cols, OP_CODE[op], vals.ctypes.data,
                     idx.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle rejected rows={rows} cols={cols} dtype={dtype} op={op}")
        return vals, idx

    def widen(self, x: np.ndarray, dtype: str) -> np.ndarray:
        """Every element of ``x`` as the oracle's scan sees it (float64)."""
        x = np.ascontiguousarray(np.asarray(x, dtype=NUMPY_STORAGE[dtype]).reshape(-1))
        out = np.empty(x.size, dtype=np.float64)
        if self._d(x.ctypes.data, DTYPE_CODE[dtype], x.size, out.ctypes.data) != 0:
            raise ValueError(dtype)
        return out


def _as_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    want = NUMPY_STORAGE[dtype]
    if x.dtype != want:
        raise TypeError(f"{dtype} data must be stored as {np.dtype(want)}, got {x.dtype}")
    if x.ndim != 2:
        raise ValueError("oracle input must be 2-D (rows, cols)")
    return np.ascontiguousarray(x)


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from this directory's source (compiled on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB)
    return _default


def argreduce_lastaxis(x: np.ndarray, dtype: str, op: str) -> np.ndarray:
    return load().argreduce_lastaxis(x, dtype, op)
