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
  last-index ops);
* the scan and the cumulative scan on arbitrary bit patterns with signalling NaNs planted,
  against the closed form on numpy's decoding of the same bits (a signalling NaN compares
  like any NaN), values passed through bit for bit.

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


# (bits type, exponent field all ones, payload bits below the quiet bit, sign bit) per format
NAN_BITS = {"f16": (np.uint16, 0x7C00, 0x01FF, 0x8000), "bf16": (np.uint16, 0x7F80, 0x003F, 0x8000),
            "f32": (np.uint32, 0x7F800000, 0x003FFFFF, 0x80000000),
            "f64": (np.uint64, 0x7FF0000000000000, 0x0007FFFFFFFFFFFF, 0x8000000000000000)}
FLOAT_NP = {"f16": np.float16, "f32": np.float32, "f64": np.float64}


def raw_bit_rows(rng, dtype: str, rows: int, cols: int) -> np.ndarray:
    """Storage array of uniformly random bit patterns in which every third entry, and
    element 0 of every other row, is a signalling NaN (quiet bit clear, random non-zero
    payload below it, random sign)."""
    bt, expo, payload, sign = NAN_BITS[dtype]
    u = rng.integers(0, np.iinfo(bt).max, size=(rows, cols), dtype=bt, endpoint=True)
    snan = (bt(expo) | rng.integers(1, payload, size=(rows, cols), dtype=bt, endpoint=True)
            | (rng.integers(0, 2, size=(rows, cols), dtype=bt) * bt(sign)))
    pick = (np.arange(cols)[None, :] % 3 == 1) | ((np.arange(rows)[:, None] % 2 == 0)
                                                   & (np.arange(cols)[None, :] == 0))
    u = np.where(pick, snan, u).astype(bt)
    quiet = bt(payload + 1)
    assert (((u[pick] & bt(expo)) == bt(expo)) & ((u[pick] & quiet) == 0)).all()
    return np.ascontiguousarray(u if dtype == "bf16" else u.view(FLOAT_NP[dtype]))


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of a storage array by numpy's own conversions; every NaN, signalling
    or quiet, becomes a NaN, which is all the closed form asks of it."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def pin_raw_bit_patterns(o, dtype: str, op: str) -> None:
    """Arbitrary bit patterns with signalling NaNs planted (leading ones included): a
    signalling NaN compares like any NaN (every comparison false), so the scan agrees with
    the closed form on numpy's decoding of the same bits."""
    rng = np.random.default_rng(71 + DTYPES.index(dtype) * 4 + OPS.index(op))
    for rows, cols in ((64, 1), (64, 2), (200, 7), (50, 64), (8, 1001)):
        x = raw_bit_rows(rng, dtype, rows, cols)
        got = o.argreduce_lastaxis(x, dtype, op)
        want = closed_form(decode(x, dtype), op)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{dtype} {op} {rows}x{cols} raw bits: row {bad[0]} -> {got[bad[0]]}, want {want[bad[0]]}"


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


# ----------------------------------------------------------------------------------------
# cumulative extremum with indices (cummax / cummin)
#
# Every position j reports the ArgMax / ArgMin scan of the prefix 0 .. j and the element
# stored at that index. The checks below compute that from outside the oracle: the closed
# form above (floats) or numpy's exact integer argmax / argmin (integers) on every prefix,
# numpy's running maximum / minimum on NaN-free data, the page's two-pass tile + carry
# recipe for the values, and the page's examples with results known by construction.

CUM_DTYPES = ("f32", "f16", "bf16", "f64", "i32", "i64")
CUM_OPS = ("max", "min")
INT_INFO = {"i32": np.iinfo(np.int32), "i64": np.iinfo(np.int64)}
INT_NP = {"i32": np.int32, "i64": np.int64}
CUM_GOLDEN = os.path.join(HERE, "golden", "cumulative_cases.json")


def int_alphabet(dtype: str) -> np.ndarray:
    i = INT_INFO[dtype]
    return np.array([i.min, i.min + 1, -1, 0, 1, i.max - 1, i.max], dtype=INT_NP[dtype])


def storage_bits(a: np.ndarray) -> np.ndarray:
    """The raw bit patterns of a storage array (so NaN payloads and zero signs compare)."""
    return np.ascontiguousarray(a).view({1: np.uint8, 2: np.uint16, 4: np.uint32,
                                         8: np.uint64}[a.dtype.itemsize])


def prefix_indices(vals: np.ndarray, dtype: str, op: str) -> np.ndarray:
    """Index of the scan over every prefix, from outside the oracle: the closed form for
    floating point, numpy's first-occurrence argmax / argmin on the exact integers."""
    rows, cols = vals.shape
    out = np.empty((rows, cols), dtype=np.int64)
    for j in range(cols):
        if dtype in INT_NP:
            f = np.argmax if op == "max" else np.argmin
            out[:, j] = f(vals[:, :j + 1], axis=1)
        else:
            out[:, j] = closed_form(vals[:, :j + 1], op)
    return out


def cum_storage(vals, dtype: str) -> np.ndarray:
    if dtype in INT_NP:
        return np.ascontiguousarray(np.asarray(vals, dtype=INT_NP[dtype]))
    return exact_storage(vals, dtype)


def check_cumulative(o, vals, dtype: str, op: str, want_idx: np.ndarray, what: str) -> None:
    x = cum_storage(vals, dtype)
    got_v, got_i = o.cumulative(x, dtype, op)
    bad = np.argwhere(got_i != want_idx)
    assert bad.size == 0, (f"{what} {dtype} {op}: index differs at {tuple(bad[0])}: "
                           f"got {got_i[tuple(bad[0])]}, want {want_idx[tuple(bad[0])]}")
    want_v = np.take_along_axis(x, want_idx, axis=1)
    assert np.array_equal(storage_bits(got_v), storage_bits(want_v)), f"{what} {dtype} {op}: values"


def pin_cum_brute_force(o, dtype: str, op: str, max_len: int = 4) -> None:
    """Every row of length 1..max_len over a special-value alphabet."""
    alpha = int_alphabet(dtype) if dtype in INT_NP else alphabet9(dtype)
    for n in range(1, max_len + 1):
        sym = np.array(list(itertools.product(range(alpha.size), repeat=n)), dtype=np.int64)
        vals = alpha[sym]
        check_cumulative(o, vals, dtype, op, prefix_indices(vals, dtype, op), f"brute len {n}")


def cum_nan_free_rows(rng, dtype: str, rows: int, cols: int, kind: str) -> np.ndarray:
    if dtype in INT_NP:
        i = INT_INFO[dtype]
        if kind == "ties":
            return rng.integers(-3, 4, size=(rows, cols)).astype(INT_NP[dtype])
        v = rng.integers(i.min, i.max, size=(rows, cols), dtype=INT_NP[dtype], endpoint=True)
        return v
    z = rng.standard_normal((rows, cols))
    v = np.clip(np.rint(4 * z), -8, 7) / 4 if kind == "ties" else z
    if dtype == "bf16":
        v = ((v.astype(np.float32).view(np.uint32) >> np.uint32(16)) << np.uint32(16)).view(np.float32)
    return v.astype({"f32": np.float32, "f16": np.float16, "bf16": np.float32,
                     "f64": np.float64}[dtype]).astype(np.float64)


def pin_cum_raw_bit_patterns(o, dtype: str, op: str) -> None:
    """Arbitrary bit patterns with signalling NaNs planted: every prefix's index is the
    closed form's on numpy's decoding of the bits, and each value is the input element at
    that index, bit for bit (a signalling NaN is passed through, not quieted)."""
    rng = np.random.default_rng(81 + CUM_DTYPES.index(dtype) * 2 + CUM_OPS.index(op))
    for rows, cols in ((64, 1), (40, 9), (6, 150)):
        x = raw_bit_rows(rng, dtype, rows, cols)
        want = prefix_indices(decode(x, dtype), dtype, op)
        got_v, got_i = o.cumulative(x, dtype, op)
        bad = np.argwhere(got_i != want)
        assert bad.size == 0, f"{dtype} {op} raw bits: index differs at {tuple(bad[0])}"
        assert np.array_equal(storage_bits(got_v), storage_bits(np.take_along_axis(x, want, axis=1))), \
            f"{dtype} {op} raw bits: values"


def pin_cum_numpy_accumulate(o, dtype: str, op: str) -> None:
    """NaN-free rows: the values are numpy's running maximum / minimum, and the index is
    the first position (within the prefix) holding that running value."""
    rng = np.random.default_rng(41 + CUM_DTYPES.index(dtype))
    acc = np.maximum.accumulate if op == "max" else np.minimum.accumulate
    for rows, cols in ((40, 1), (17, 130), (3, 700)):
        for kind in ("normal", "ties"):
            v = cum_nan_free_rows(rng, dtype, rows, cols, kind)
            x = cum_storage(v, dtype)
            got_v, got_i = o.cumulative(x, dtype, op)
            run = acc(v, axis=1)
            num = got_v.astype(np.float64) if dtype == "bf16" else got_v
            if dtype == "bf16":
                num = (got_v.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
            assert np.array_equal(num, run), f"{dtype} {op} {kind}: values vs numpy accumulate"
            pos = np.arange(cols)
            for j in range(cols):
                first = np.argmax((v == run[:, j:j + 1]) & (pos <= j), axis=1)
                assert np.array_equal(got_i[:, j], first), f"{dtype} {op} {kind}: index at {j}"


def pin_cum_two_pass(o, dtype: str, op: str) -> None:
    """The page's two-pass recipe for the values of a long 1-D scan: running extremum
    within tiles, running extremum of the tile ends shifted by one tile (the carry, the
    format's lowest (highest) value first), and the elementwise extremum of the two. The
    page reports it bit-equal to the one-pass scan (on NaN-free data)."""
    rng = np.random.default_rng(53 + CUM_DTYPES.index(dtype))
    tiles, width = 64, 48
    v = cum_nan_free_rows(rng, dtype, 1, tiles * width, "ties")[0]
    acc = np.maximum.accumulate if op == "max" else np.minimum.accumulate
    pick = np.maximum if op == "max" else np.minimum
    if dtype in INT_NP:
        edge = INT_INFO[dtype].min if op == "max" else INT_INFO[dtype].max
    else:
        edge = -np.inf if op == "max" else np.inf
    part = acc(v.reshape(tiles, width), axis=1)
    carry = acc(part[:, -1])
    carry = np.concatenate([np.array([edge], dtype=v.dtype), carry[:-1]])
    want = pick(part, carry[:, None]).reshape(-1)
    got_v, _ = o.cumulative(cum_storage(v[None, :], dtype), dtype, op)
    num = got_v[0]
    if dtype == "bf16":
        num = (num.astype(np.uint32) << np.uint32(16)).view(np.float32)
    assert np.array_equal(num.astype(v.dtype), want), f"{dtype} {op}: two-pass recipe"


def pin_cum_page_examples(o) -> None:
    """The page's own data, with results known by construction: cummax / cummin of an
    int64 arange of 65536 elements (reproduction script), and the document-start forward
    fill cummax(is_boundary * positions) of its real-impact section."""
    n = 65536
    a = np.arange(n, dtype=np.int64)[None, :]
    v, i = o.cumulative(a, "i64", "max")
    assert np.array_equal(v[0], a[0]) and np.array_equal(i[0], a[0]), "arange cummax"
    v, i = o.cumulative(a, "i64", "min")
    assert not v.any() and not i.any(), "arange cummin"
    rng = np.random.default_rng(61)
    starts = np.sort(rng.choice(np.arange(1, n), size=40, replace=False))
    x = np.zeros(n, dtype=np.int64)
    x[starts] = starts
    want = np.zeros(n, dtype=np.int64)  # start of the document holding each position
    for s in starts:
        want[s:] = s
    v, i = o.cumulative(x[None, :], "i64", "max")
    assert np.array_equal(v[0], want), "document starts: values"
    assert np.array_equal(i[0], want), "document starts: indices (a start is its own index)"


def pin_cum_fixed_cases(o, section: str = "cases") -> None:
    with open(CUM_GOLDEN) as f:
        cases = json.load(f)[section]
    for case in cases:
        for dtype in case["dtypes"]:
            for spec, want in zip(case["rows"], case["expect"]):
                if dtype in INT_NP:
                    row = np.array([int(s) for s in spec], dtype=object).astype(INT_NP[dtype])
                else:
                    row = golden_row(spec, dtype)
                check_cumulative(o, row[None, :], dtype, case["op"],
                                 np.array([want], dtype=np.int64), case["name"])


def pin_cum_rejects(o) -> None:
    for bad in ((np.zeros((2, 0), np.float32), "f32", "max"), (np.zeros((2, 3), np.float32), "f32", "max_last")):
        try:
            o.cumulative(*bad)
        except ValueError:
            continue
        raise AssertionError(f"the oracle must refuse {bad[1]} {bad[2]} of shape {bad[0].shape}")


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
            pins.append((f"bits_{dtype}_{op}", lambda d=dtype, p=op: pin_raw_bit_patterns(o, d, p)))
    pins += [("cum_fixed_cases", lambda: pin_cum_fixed_cases(o, "cases")),
             ("cum_readings", lambda: pin_cum_fixed_cases(o, "readings")),
             ("cum_page_examples", lambda: pin_cum_page_examples(o)),
             ("cum_rejects", lambda: pin_cum_rejects(o))]
    for dtype in CUM_DTYPES:
        for op in CUM_OPS:
            pins.append((f"cum_brute_{dtype}_{op}",
                         lambda d=dtype, p=op: pin_cum_brute_force(o, d, p, 3 if fast else 4)))
            pins.append((f"cum_numpy_{dtype}_{op}", lambda d=dtype, p=op: pin_cum_numpy_accumulate(o, d, p)))
            pins.append((f"cum_two_pass_{dtype}_{op}", lambda d=dtype, p=op: pin_cum_two_pass(o, d, p)))
            if dtype not in INT_NP:
                pins.append((f"cum_bits_{dtype}_{op}",
                             lambda d=dtype, p=op: pin_cum_raw_bit_patterns(o, d, p)))
    return pins
