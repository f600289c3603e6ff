"""Helpers of the GPU parity tests: move storage arrays to the device, call the HIP library
through its C ABI, and name every case on stdout before it touches the GPU."""
from __future__ import annotations

import sys

import numpy as np

import argmin_reduction_wide_amd.binding as B


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str, offset_elems: int = 0):
    """A contiguous CUDA tensor holding ``arr``; with ``offset_elems`` > 0 its data starts
    that many elements into a larger allocation (misaligned row starts)."""
    import torch

    flat = np.ascontiguousarray(arr).reshape(-1)
    if dtype == "bf16":
        host = torch.from_numpy(flat.view(np.int16).copy()).view(torch.bfloat16)
    else:
        host = torch.from_numpy(flat.copy())
    if offset_elems:
        buf = torch.empty(flat.size + offset_elems, dtype=host.dtype, device="cuda")
        t = buf[offset_elems:offset_elems + flat.size]
        t.copy_(host.to("cuda"))
    else:
        t = host.to("cuda")
    return t.view(arr.shape)


def run(t, dtype: str, op: str, scratch=None, scratch_offset: int = 0, out=None):
    """Call argreduce_lastaxis on a 2-D CUDA tensor; returns (status, int64 numpy result)."""
    import torch

    rows, cols = t.shape
    need = B.argreduce_scratch_bytes(rows, cols, dtype)
    assert need != B.SIZE_MAX
    if scratch is None and need:
        scratch = torch.empty(need + scratch_offset, dtype=torch.uint8, device="cuda")
    if out is None:
        out = torch.full((rows,), -7, dtype=torch.int64, device="cuda")
    sptr = scratch.data_ptr() + scratch_offset if scratch is not None else 0
    sbytes = scratch.numel() - scratch_offset if scratch is not None else 0
    stream = torch.cuda.current_stream().cuda_stream
    rc = B.argreduce_lastaxis(t.data_ptr(), dtype, rows, cols, op, out.data_ptr(), sptr, sbytes,
                              stream)
    torch.cuda.synchronize()
    return rc, out.cpu().numpy()


def check(oracle_lib, arr: np.ndarray, dtype: str, op: str, what: str, **kw) -> np.ndarray:
    """Run the library on ``arr`` and require bit-exact agreement with the oracle."""
    announce(f"{what} dtype={dtype} op={op} shape={arr.shape} {kw}")
    offset = kw.pop("offset_elems", 0)
    t = to_device(arr, dtype, offset)
    rc, got = run(t, dtype, op, **kw)
    assert rc == 0, f"{what}: status {rc}"
    want = oracle_lib.argreduce_lastaxis(arr, dtype, op)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{what} {dtype} {op} {arr.shape}: {bad.size} rows differ; first row "
                           f"{bad[0]}: got {got[bad[0]]}, oracle {want[bad[0]]}")
    return got
