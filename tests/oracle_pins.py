"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin takes an ``oracle.Oracle`` and raises ``AssertionError`` when that oracle
disagrees with something fixed from outside it:

* the element decoders against numpy's and torch's own format conversions (library
  routines), over every f16 and bf16 bit pattern and a large sample of f32 / f64 patterns;
* the scan against an independently written two-pass closed form (drop NaNs, take the
  extremum, take its first position; a leading NaN gives 0), by brute force over every row
  of length 1..5 drawn from a 9-symbol alphabet of special values;
* the scan against the fixed cases the ONNX Runtime pages state (tests/golden);
* the scan against numpy.argmax / numpy.argmin, which return the first occurrence of the
  extremum and agree with the definition on NaN-free rows (on reversed rows for the
  last-index ops).

The closed form is derived as follows. If element 0 is NaN the scan never moves (every
comparison with NaN is false), so the result is 0. Otherwise the running best is never
NaN, a NaN element is never taken, and the strict comparison moves only to a strictly
better element; so the scan ends at the first position holding the extremum of the
non-NaN elements (which include element 0). -0 and +0 compare equal; -inf and +inf are
ordinary extremes. With the non-strict comparison of the last-index ops the scan also
moves to equal elements, so it ends at the LAST position holding that extremum (and still
at 0 when element 0 is NaN, since every comparison with the NaN running best is false).

These functions are shared by tests/test_oracle_pins.py (run on the real oracle) and by
tests/test_oracle_mutants.py (run on deliberately broken copies of it, each of which must
fail at least one pin).
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "pages_fixed_cases.json")
DTYPES = ("f32", "f16", "bf16", "f64")
OPS = ("max", "min", "max_last", "min_last")

MIN_SUBNORMAL = {"f32": 2.0 ** -149, "f16": 2.0 ** -24, "bf16": 2.0 ** -133, "f64": 2.0 ** -1074}
MAX_FINITE = {"f32": float(np.finfo(np.float32).max), "f16": 65504.0,
              "bf16": float.fromhex("0x1.fep127"), "f64": float(np.finfo(np.float64).max)}


def exact_storage(values, dtype: str) -> np.ndarray:
    """Storage array for float64 values that are exactly representable in ``dtype``."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == "f64":
        return np.ascontiguousarray(v)
    if dtype == "f32":
        s = v.astype(np.float32)
        assert np.array_equal(s.astype(np.float64), v, equal_nan=True)
        return np.ascontiguousarray(s)
    if dtype == "f16":
        s = v.astype(np.float16)
        assert np.array_equal(s.astype(np.float64), v, equal_nan=True)
        return np.ascontiguousarray(s)
    # bf16 = the upper 16 bits of the binary32 encoding; exact values have zero low bits.
    u = np.ascontiguousarray(v.astype(np.float32)).view(np.uint32)
    assert not (u[~np.isnan(v)] & np.uint32(0xFFFF)).any(), "value not exact in bf16"
    return np.ascontiguousarray((u >> np.uint32(16)).astype(np.uint16))


def closed_form(values: np.ndarray, op: str) -> np.ndarray:
    """First (last, for the *_last ops) position of the extremum of the non-NaN elements;
    0 when element 0 is NaN."""
    v = np.asarray(values, dtype=np.float64)
    nan = np.isnan(v)
    if op in ("max", "max_last"):
        ext = np.where(nan, -np.inf, v).max(axis=1)
    else:
        ext = np.where(nan, np.inf, v).min(axis=1)
    hit = v == ext[:, None]
    if op.endswith("_last"):
        pos = v.shape[1] - 1 - hit[:, ::-1].argmax(axis=1)
    else:
        pos = hit.argmax(axis=1)
    return np.where(nan[:, 0], 0, pos).astype(np.int64)


def symbol(s, dtype: str) -> float:
    if isinstance(s, (int, float)):
        return float(s)
    table = {"nan": math.nan, "inf": math.inf, "-inf": -math.inf, "-0.0": -0.0,
             "max": MAX_FINITE[dtype], "-max": -MAX_FINITE[dtype],
             "minsub": MIN_SUBNORMAL[dtype], "-minsub": -MIN_SUBNORMAL[dtype]}
    return table[s]


def golden_row(spec, dtype: str) -> np.ndarray:
    if isinstance(spec, dict):
        row = np.full(spec["cols"], symbol(spec["fill"], dtype), dtype=np.float64)
        for k, val in spec["set"].items():
            row[int(k)] = symbol(val, dtype)
        return row
    return np.array([symbol(s, dtype) for s in spec], dtype=np.float64)


def golden_cases(section: str = "cases"):
    with open(GOLDEN) as f:
        return json.load(f)[section]


# ----------------------------------------------------------------------------------------
# pins


def pin_widen_f16(o) -> None:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.widen(bits.view(np.float16), "f16")
    want = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want)), "f16 NaN set differs from numpy"
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]), "f16 decode differs from numpy"
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok])), "f16 sign differs"


def pin_widen_bf16(o) -> None:
    import torch

    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.widen(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want)), "bf16 NaN set differs from torch"
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]), "bf16 decode differs from torch"
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok])), "bf16 sign differs"


def pin_widen_f32_f64(o) -> None:
    rng = np.random.default_rng(11)
    b32 = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    b32[:8] = [0, 0x80000000, 1, 0x80000001, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F7FFFFF]
    got = o.widen(b32.view(np.float32), "f32")
    want = b32.view(np.float32).astype(np.float64)
    assert np.array_equal(got, want, equal_nan=True), "f32 widening differs from numpy"
    assert np.array_equal(np.signbit(got), np.signbit(want)), "f32 sign differs"
    b64 = rng.integers(0, 2 ** 63, size=100_000, dtype=np.int64).view(np.uint64)
    b64 ^= rng.integers(0, 2, size=b64.size).astype(np.uint64) << np.uint64(63)
    got = o.widen(b64.view(np.float64), "f64")
    want = b64.view(np.float64)
    assert np.array_equal(got, want, equal_nan=True), "f64 read differs"


def alphabet9(dtype: str) -> np.ndarray:
    s = MIN_SUBNORMAL[dtype]
    return np.array([math.nan, -math.inf, -1.0, -s, -0.0, 0.0, s, 1.0, math.inf])


def pin_brute_force(o, dtype: str, op: str, max_len: int = 5) -> None:
    """Every row of length 1..max_len over the 9-symbol alphabet, one call per length."""
    alpha = alphabet9(dtype)
    for n in range(1, max_len + 1):
        sym = np.array(list(itertools.product(range(alpha.size), repeat=n)), dtype=np.int64)
        vals = alpha[sym]
        got = o.argreduce_lastaxis(exact_storage(vals, dtype), dtype, op)
        want = closed_form(vals, op)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"{dtype} {op} len {n}: {bad.size} rows differ, e.g. "
                               f"{vals[bad[0]].tolist()} -> {got[bad[0]]}, want {want[bad[0]]}")


def pin_fixed_cases(o, section: str = "cases") -> None:
    for case in golden_cases(section):
        for dtype in case["dtypes"]:
            for spec, want in zip(case["rows"], case["expect"]):
                row = golden_row(spec, dtype)
                got = o.argreduce_lastaxis(exact_storage(row[None, :], dtype), dtype, case["op"])
                assert got[0] == want, f"{case['name']} {dtype}: got {got[0]}, want {want}"


def pin_numpy_first_occurrence(o, dtype: str, op: str) -> None:
    """NaN-free rows (continuous values and 16-level ties): numpy's argmax/argmin agree."""
    rng = np.random.default_rng(23)
    for rows, cols in ((257, 1), (64, 3), (33, 130), (5, 4099)):
        for kind in ("normal", "ties"):
            z = rng.standard_normal((rows, cols))
            v = np.clip(np.rint(4 * z), -8, 7) / 4 if kind == "ties" else z
            if dtype == "bf16":
                v = v.astype(np.float32)
                v = ((v.view(np.uint32) >> np.uint32(16)) << np.uint32(16)).view(np.float32)
            v = v.astype({"f32": np.float32, "f16": np.float16, "bf16": np.float32,
                          "f64": np.float64}[dtype]).astype(np.float64)
            f = np.argmax if op.startswith("max") else np.argmin
            if op.endswith("_last"):
                want = cols - 1 - f(v[:, ::-1], axis=1)
            else:
                want = f(v, axis=1)
            got = o.argreduce_lastaxis(exact_storage(v, dtype), dtype, op)
            assert np.array_equal(got, want), f"{dtype} {op} {rows}x{cols} {kind} vs numpy"


def pin_axis(o, dtype: str, op: str) -> None:
    """The middle-axis scan against the closed form applied to the transposed data, and
    against the last-axis scan when inner == 1."""
    rng = np.random.default_rng(31 + DTYPES.index(dtype) * 4 + OPS.index(op))
    alpha = alphabet9(dtype)
    for outer, length, inner in ((1, 1, 1), (2, 5, 3), (3, 17, 1), (1, 64, 33), (4, 9, 70),
                                 (2, 300, 5)):
        vals = alpha[rng.integers(0, alpha.size, size=(outer, length, inner))]
        if length > 5:  # mostly ordinary values, with ties, so rows have a real extremum
            q = np.clip(np.rint(4 * rng.standard_normal((outer, length, inner))), -8, 7) / 4
            keep = rng.random((outer, length, inner)) < 0.9
            vals = np.where(keep, q, vals)
        got = o.argreduce_axis(exact_storage(vals, dtype), dtype, op)
        rows = np.moveaxis(vals, 1, 2).reshape(outer * inner, length)
        want = closed_form(rows, op).reshape(outer, inner)
        assert np.array_equal(got, want), f"axis {dtype} {op} {vals.shape}"
        if inner == 1:
            last = o.argreduce_lastaxis(exact_storage(vals[:, :, 0], dtype), dtype, op)
            assert np.array_equal(got[:, 0], last), f"axis vs last axis {dtype} {op}"
    v = rng.standard_normal((3, 40, 7))
    if dtype == "bf16":
        v = ((v.astype(np.float32).view(np.uint32) >> np.uint32(16)) << np.uint32(16)).view(np.float32)
    v = v.astype({"f32": np.float32, "f16": np.float16, "bf16": np.float32,
                  "f64": np.float64}[dtype]).astype(np.float64)
    f = np.argmax if op.startswith("max") else np.argmin
    want = (v.shape[1] - 1 - f(v[:, ::-1, :], axis=1)) if op.endswith("_last") else f(v, axis=1)
    assert np.array_equal(o.argreduce_axis(exact_storage(v, dtype), dtype, op), want), "axis vs numpy"


def pin_rejects_empty_rows(o) -> None:
    try:
        o.argreduce_lastaxis(np.zeros((3, 0), dtype=np.float32), "f32", "max")
    except ValueError:
        return
    raise AssertionError("an empty row has no index; the oracle must refuse cols == 0")


def all_pins(o, fast: bool = False):
    """(name, thunk) for every pin; ``fast`` trims the brute force to length 4."""
    max_len = 4 if fast else 5
    pins = [("widen_f16", lambda: pin_widen_f16(o)),
            ("widen_bf16", lambda: pin_widen_bf16(o)),
            ("widen_f32_f64", lambda: pin_widen_f32_f64(o)),
            ("fixed_cases", lambda: pin_fixed_cases(o, "cases")),
            ("readings", lambda: pin_fixed_cases(o, "readings")),
            ("rejects_empty", lambda: pin_rejects_empty_rows(o))]
    for dtype in DTYPES:
        for op in OPS:
            pins.append((f"brute_{dtype}_{op}",
                         lambda d=dtype, p=op: pin_brute_force(o, d, p, max_len)))
            pins.append((f"numpy_{dtype}_{op}",
                         lambda d=dtype, p=op: pin_numpy_first_occurrence(o, d, p)))
            pins.append((f"axis_{dtype}_{op}", lambda d=dtype, p=op: pin_axis(o, d, p)))
    return pins
