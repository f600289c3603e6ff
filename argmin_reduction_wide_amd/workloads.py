"""Seeded synthetic inputs for the last-axis ArgMax / ArgMin workloads.

This module only draws inputs. It holds no part of the reduction: it never compares
elements to find an extremum. Where a workload plants structure whose answer is known
in advance (a duplicated maximum, a constant row, extrema in the ragged tail, a leading
NaN, ...), the expected index is known from how the row was built, and is returned next
to the data as ``planted``.

The shapes and value distributions are those of the workloads measured on the
"[CUDA] Parallelize ArgMax/ArgMin over wide last axes" page (Description, Results table:
[1, 32000], [1, 202048], [32, 202048], [4096, 4096], [65536, 1024], [65536, 64]); the
values themselves are synthetic (the page's sampler logits are not available), drawn as
follows:

* every draw is float64 from ``numpy.random.default_rng(seed)`` (PCG64) and is rounded once
  to the element format: numpy's ``astype`` (round to nearest even) for f32 and f16; for
  bf16 the f32 value is rounded to nearest even on its bit pattern;
* row subsets that carry planted structure are disjoint, taken from one
  ``rng.permutation``; "p% of rows" means ceil(p/100 * rows).

Storage: f32 -> numpy float32, f16 -> numpy float16, bf16 -> numpy uint16 holding the
bfloat16 bit patterns, f64 -> numpy float64; always C-contiguous (rows, cols).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "f64": np.float64,
           "i32": np.int32, "i64": np.int64}
ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2, "f64": 8, "i32": 4, "i64": 8}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the bits.

    NaN inputs map to the quiet NaN 0x7FC0 with the input's sign bit.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    rounded = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        sign = ((u >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
        rounded = np.where(nan, sign | np.uint16(0x7FC0), rounded).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (used for display and checks)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(values: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 ``values`` once to ``dtype`` and return the storage array."""
    values = np.asarray(values, dtype=np.float64)
    if dtype == "bf16":
        return np.ascontiguousarray(f32_to_bf16_bits(values.astype(np.float32)))
    return np.ascontiguousarray(values.astype(STORAGE[dtype]))


def _count(pct: float, rows: int) -> int:
    return int(math.ceil(pct / 100.0 * rows - 1e-9))


@dataclass
class Workload:
    """One seeded input tensor plus what its construction fixes about the answer."""

    name: str
    dtype: str
    ops: tuple
    data: np.ndarray
    seed: int
    recipe: str
    planted: dict = field(default_factory=dict)  # op -> {row: expected index}
    # For a reduction over a middle axis: (outer, len, inner); data is then stored as
    # (outer, len * inner) and the reduced axis is `len`.
    axis_shape: tuple | None = None
    # "argreduce" (ArgMax / ArgMin, one index per row) or "scan" (cummax / cummin: a value
    # and an index per element)
    kind: str = "argreduce"
    # Set for inputs too large to hold on the host: ((rows, cols), {flat index: value});
    # `data` is then one block that fills the tensor by repetition (see device_data).
    tiled: tuple | None = None

    @property
    def rows(self) -> int:
        return int(self.tiled[0][0] if self.tiled else self.data.shape[0])

    @property
    def cols(self) -> int:
        return int(self.tiled[0][1] if self.tiled else self.data.shape[1])

    @property
    def nbytes(self) -> int:
        return self.rows * self.cols * ITEMSIZE[self.dtype]


def c1_row32000_f32(seed: int = 1, cols: int = 32000) -> Workload:
    """ArgMax f32 [1, 32000]: iid N(0,1); the row maximum appears twice, at j and at a later k.

    The maximum is planted as the value 8.0 (beyond every N(0,1) draw of this size; the
    construction asserts that no draw reaches it), so the expected ArgMax is j.
    """
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((1, cols))
    j = int(rng.integers(0, cols - 1))
    k = int(rng.integers(j + 1, cols))
    assert not (v >= 8.0).any()
    v[0, j] = v[0, k] = 8.0
    return Workload(
        name=f"argmax_f32_1x{cols}", dtype="f32", ops=("max",), data=to_storage(v, "f32"),
        seed=seed, planted={"max": {0: j}},
        recipe=f"iid N(0,1) f64 -> f32; value 8.0 planted at j={j} and k={k} > j",
    )


def c2_row202048_f32(seed: int = 2, rows: int = 1, cols: int = 202048) -> Workload:
    """ArgMax and ArgMin f32 [1, 202048] ('vocab-size sampler logits'): iid N(0, 4) (sigma 2)."""
    rng = np.random.default_rng(seed)
    v = rng.normal(0.0, 2.0, size=(rows, cols))
    return Workload(
        name=f"argmax_argmin_f32_{rows}x{cols}", dtype="f32", ops=("max", "min"),
        data=to_storage(v, "f32"), seed=seed,
        recipe="iid N(0, 4) read as variance 4 (sigma = 2), f64 -> f32",
    )


def c3_rows32_f16_bf16(dtype: str, seed: int = 3, rows: int = 32, cols: int = 202048) -> Workload:
    """ArgMax/ArgMin f16 or bf16 [32, 202048]: iid N(0,1) rounded to the format (many ties).

    1% of rows are constant (one N(0,1) draw; expected index 0 for both ops); 1% of rows
    carry +8 at cols-1 and -8 at cols-2, the last positions of every ragged tail (expected
    ArgMax cols-1, ArgMin cols-2; no N(0,1) draw of this size reaches |8|, asserted).
    """
    assert dtype in ("f16", "bf16")
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols))
    perm = rng.permutation(rows)
    n1 = _count(1, rows)
    const_rows = perm[:n1]
    tail_rows = perm[n1:2 * n1]
    for r in const_rows:
        v[r, :] = rng.standard_normal()
    assert not (np.abs(v[tail_rows]) >= 8.0).any()
    for r in tail_rows:
        v[r, cols - 1] = 8.0
        v[r, cols - 2] = -8.0
    planted = {"max": {}, "min": {}}
    for r in const_rows:
        planted["max"][int(r)] = 0
        planted["min"][int(r)] = 0
    for r in tail_rows:
        planted["max"][int(r)] = cols - 1
        planted["min"][int(r)] = cols - 2
    return Workload(
        name=f"argmax_argmin_{dtype}_{rows}x{cols}", dtype=dtype, ops=("max", "min"),
        data=to_storage(v, dtype), seed=seed, planted=planted,
        recipe=(f"iid N(0,1) f64 -> {dtype}; rows {sorted(map(int, const_rows))} constant; "
                f"rows {sorted(map(int, tail_rows))} get +8 at cols-1 and -8 at cols-2"),
    )


def c4_square_f32_f64(dtype: str, seed: int = 4, rows: int = 4096, cols: int = 4096) -> Workload:
    """ArgMax f32 or f64 [4096, 4096]: iid U(-1,1) (f32 is the f64 draws rounded).

    2% of rows get 1-4 entries of +inf or -inf (sign uniform) at uniform distinct
    positions; where one is +inf the expected ArgMax is the first +inf. 1% of rows start
    with NaN (expected 0). 1% of rows are all -inf (expected 0).
    """
    assert dtype in ("f32", "f64")
    rng = np.random.default_rng(seed)
    v = rng.uniform(-1.0, 1.0, size=(rows, cols))
    perm = rng.permutation(rows)
    n_inf, n1 = _count(2, rows), _count(1, rows)
    inf_rows = perm[:n_inf]
    nan_rows = perm[n_inf:n_inf + n1]
    ninf_rows = perm[n_inf + n1:n_inf + 2 * n1]
    planted = {"max": {}}
    for r in inf_rows:
        m = int(rng.integers(1, 5))
        pos = rng.choice(cols, size=m, replace=False)
        sgn = rng.integers(0, 2, size=m)
        for p, s in zip(pos, sgn):
            v[r, p] = math.inf if s else -math.inf
        pos_plus = [int(p) for p, s in zip(pos, sgn) if s]
        if pos_plus:
            planted["max"][int(r)] = min(pos_plus)
    for r in nan_rows:
        v[r, 0] = math.nan
        planted["max"][int(r)] = 0
    for r in ninf_rows:
        v[r, :] = -math.inf
        planted["max"][int(r)] = 0
    return Workload(
        name=f"argmax_{dtype}_{rows}x{cols}", dtype=dtype, ops=("max",),
        data=to_storage(v, dtype), seed=seed, planted=planted,
        recipe=("iid U(-1,1) f64 (f32 = the same draws rounded); 2% rows +-inf at 1-4 "
                "uniform positions, 1% rows NaN at column 0, 1% rows all -inf"),
    )


def quantised_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) quantised to 16 levels: clip(round(4 z), -8, 7) / 4, exact in f16 and f32."""
    z = rng.standard_normal(shape)
    return np.clip(np.rint(4.0 * z), -8.0, 7.0) / 4.0


def c5a_many_rows_f32(seed: int = 5, rows: int = 65536, cols: int = 1024) -> Workload:
    """ArgMin f32 [65536, 1024]: N(0,1) quantised to 16 levels (frequent ties)."""
    rng = np.random.default_rng(seed)
    return Workload(
        name=f"argmin_f32_{rows}x{cols}", dtype="f32", ops=("min",),
        data=to_storage(quantised_normal(rng, (rows, cols)), "f32"), seed=seed,
        recipe="N(0,1) quantised to 16 levels clip(round(4z),-8,7)/4, f32",
    )


def c5b_narrow_rows_f16(seed: int = 6, rows: int = 65536, cols: int = 64) -> Workload:
    """ArgMax f16 [65536, 64]: N(0,1) quantised to 16 levels (frequent ties)."""
    rng = np.random.default_rng(seed)
    return Workload(
        name=f"argmax_f16_{rows}x{cols}", dtype="f16", ops=("max",),
        data=to_storage(quantised_normal(rng, (rows, cols)), "f16"), seed=seed,
        recipe="N(0,1) quantised to 16 levels clip(round(4z),-8,7)/4, f16",
    )


def axis_many_outputs_f32(seed: int = 7, outer: int = 64, length: int = 4096,
                          inner: int = 256) -> Workload:
    """ArgMax f32 over the middle axis of [64, 4096, 256]: 16384 outputs, each over 4096
    elements 1 KiB apart; N(0,1) quantised to 16 levels (frequent ties)."""
    rng = np.random.default_rng(seed)
    v = quantised_normal(rng, (outer, length * inner))
    return Workload(
        name=f"argmax_f32_axis1_{outer}x{length}x{inner}", dtype="f32", ops=("max",),
        data=to_storage(v, "f32"), seed=seed, axis_shape=(outer, length, inner),
        recipe="N(0,1) quantised to 16 levels, f32, reduced over the middle axis",
    )


def axis_few_outputs_f32(seed: int = 8, outer: int = 1, length: int = 1 << 20,
                         inner: int = 32) -> Workload:
    """ArgMax f32 over the middle axis of [1, 1048576, 32]: 32 outputs over a long axis
    (a column reduction of a tall, narrow matrix); N(0,1) quantised to 16 levels."""
    rng = np.random.default_rng(seed)
    v = quantised_normal(rng, (outer, length * inner))
    return Workload(
        name=f"argmax_f32_axis1_{outer}x{length}x{inner}", dtype="f32", ops=("max",),
        data=to_storage(v, "f32"), seed=seed, axis_shape=(outer, length, inner),
        recipe="N(0,1) quantised to 16 levels, f32, reduced over the middle axis",
    )


def axis_element_loads_f16(seed: int = 15, outer: int = 4, length: int = 16384,
                           inner: int = 1001) -> Workload:
    """ArgMax fp16 over the middle axis of [4, 16384, 1001]: rows of 1001 halves (2002
    bytes) are not whole 16-byte vectors, so every lane loads one element per position;
    N(0,1) quantised to 16 levels."""
    rng = np.random.default_rng(seed)
    v = quantised_normal(rng, (outer, length * inner))
    return Workload(
        name=f"argmax_f16_axis1_{outer}x{length}x{inner}", dtype="f16", ops=("max",),
        data=to_storage(v, "f16"), seed=seed, axis_shape=(outer, length, inner),
        recipe="N(0,1) quantised to 16 levels, f16, reduced over the middle axis (element loads)",
    )


# ----------------------------------------------------------------------------------------
# cummax / cummin workloads. The PaddlePaddle issue on the cummax/cummin kernel measures
# [1, N] and [rows, 65536 / rows] int64 scans along the last axis (reproduction A, B), a
# dtype table at [1, 65536] (F), and names its real use: cummax(is_boundary * positions)
# over a [65536] int64 tensor in long-context pre-training (real impact). Its inputs are
# arange tensors; seeded random values stand in here, so that ties, new extrema and (for
# floats) both ops are exercised. The long row and the many-row shape are ours: they make
# the scan bandwidth-bound.


def scan_doc_starts_i64(seed: int = 9, n: int = 65536, mean_doc: int = 2048) -> Workload:
    """cummax of is_boundary * positions over one [1, 65536] int64 row: each position gets
    the start of its document. Boundaries: position 0 and a Bernoulli(1/mean_doc) draw at
    every other position. Expected by construction: values = indices = the last boundary at
    or before each position."""
    rng = np.random.default_rng(seed)
    is_b = rng.random(n) < 1.0 / mean_doc
    is_b[0] = True
    x = (is_b.astype(np.int64) * np.arange(n, dtype=np.int64))[None, :]
    starts = np.flatnonzero(is_b)
    return Workload(
        name=f"cummax_i64_doc_starts_1x{n}", dtype="i64", ops=("max",), data=np.ascontiguousarray(x),
        seed=seed, kind="scan", planted={"starts": starts},
        recipe=f"is_boundary (position 0, then Bernoulli(1/{mean_doc})) * positions, int64",
    )


def scan_rows_i64(rows: int, cols: int, seed: int = 10) -> Workload:
    """cummax / cummin int64 over [rows, cols] (65536 elements in the page's table):
    uniform draws in [-2^62, 2^62)."""
    rng = np.random.default_rng(seed + rows)
    x = rng.integers(-(1 << 62), 1 << 62, size=(rows, cols), dtype=np.int64)
    return Workload(name=f"cummax_cummin_i64_{rows}x{cols}", dtype="i64", ops=("max", "min"),
                    data=np.ascontiguousarray(x), seed=seed + rows, kind="scan",
                    recipe="uniform int64 in [-2^62, 2^62)")


def scan_row_65536(dtype: str, seed: int = 11, n: int = 65536) -> Workload:
    """cummax of one [1, 65536] row per format of the page's dtype table: N(0,1) for
    floating point, uniform int32 for i32."""
    rng = np.random.default_rng(seed)
    if dtype == "i32":
        x = rng.integers(np.iinfo(np.int32).min, np.iinfo(np.int32).max, size=(1, n),
                         dtype=np.int32, endpoint=True)
        recipe = "uniform int32"
    else:
        x = to_storage(rng.standard_normal((1, n)), dtype)
        recipe = f"iid N(0,1) -> {dtype}"
    return Workload(name=f"cummax_{dtype}_1x{n}", dtype=dtype, ops=("max",),
                    data=np.ascontiguousarray(x), seed=seed, kind="scan", recipe=recipe)


def scan_long_row_f32(seed: int = 12, n: int = 1 << 24) -> Workload:
    """cummax / cummin f32 over one row of 2^24 elements (64 MiB in, 192 MiB out)."""
    rng = np.random.default_rng(seed)
    return Workload(name=f"cummax_cummin_f32_1x{n}", dtype="f32", ops=("max", "min"),
                    data=to_storage(rng.standard_normal((1, n)), "f32"), seed=seed, kind="scan",
                    recipe="iid N(0,1) -> f32")


def scan_many_rows_f32(seed: int = 13, rows: int = 4096, cols: int = 4096) -> Workload:
    """cummax f32 over [4096, 4096]: one tile per row, no look-back."""
    rng = np.random.default_rng(seed)
    return Workload(name=f"cummax_f32_{rows}x{cols}", dtype="f32", ops=("max",),
                    data=to_storage(rng.standard_normal((rows, cols)), "f32"), seed=seed,
                    kind="scan", recipe="iid N(0,1) -> f32")


def wide_row_f16(seed: int = 14, cols: int = (1 << 31) + 4096) -> Workload:
    """ArgMax / ArgMin fp16 over one row of 2^31 + 4096 elements (4 GiB), wider than
    INT32_MAX: a seeded block of 2^20 N(0,1) draws repeated over the row, with +8 planted at
    2^31 + 17 and 2^31 + 100 and -8 at 5 and 2^31 + 4000 (beyond every draw). Expected by
    construction: ArgMax 2^31 + 17, ArgMin 5. Only the block is held on the host;
    ``device_data`` builds the row on the GPU."""
    rng = np.random.default_rng(seed)
    block = to_storage(rng.standard_normal(1 << 20), "f16")
    assert np.abs(block.astype(np.float32)).max() < 8.0
    plants = {(1 << 31) + 17: 8.0, (1 << 31) + 100: 8.0, 5: -8.0, (1 << 31) + 4000: -8.0}
    return Workload(name=f"argmax_argmin_f16_1x{cols}", dtype="f16", ops=("max", "min"),
                    data=block[None, :], seed=seed,
                    planted={"max": {0: (1 << 31) + 17}, "min": {0: 5}},
                    recipe="2^20 seeded N(0,1) f16 draws repeated over the row; +-8 planted",
                    tiled=((1, cols), plants))


def device_data(w: Workload, device: str = "cuda"):
    """The workload's input as a contiguous torch tensor on ``device``: a copy of ``data``,
    or, for a tiled workload, its block repeated to the full shape on the device with the
    planted values set (no host array of the full size)."""
    import torch

    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "f64": torch.float64, "i32": torch.int32, "i64": torch.int64}[w.dtype]
    flat = np.ascontiguousarray(w.data).reshape(-1)
    host = (torch.from_numpy(flat.view(np.int16).copy()).view(torch.bfloat16)
            if w.dtype == "bf16" else torch.from_numpy(flat.copy()))
    if w.tiled is None:
        return host.to(device).view(w.data.shape)
    (rows, cols), plants = w.tiled
    block = host.to(device)
    n = rows * cols
    out = torch.empty(n, dtype=tdt, device=device)
    whole = n // block.numel() * block.numel()
    out[:whole].view(-1, block.numel()).copy_(block.expand(whole // block.numel(), -1))
    out[whole:].copy_(block[:n - whole])
    for k, v in plants.items():
        out[k] = v
    return out.view(rows, cols)


def random_int_rows(rng: np.random.Generator, rows: int, cols: int, dtype: str, kind: str) -> np.ndarray:
    """A (rows, cols) int32 / int64 array: "ties" (values in [-3, 3]), "full" (the whole
    range, extremes included) or "constant"."""
    t = STORAGE[dtype]
    info = np.iinfo(t)
    if kind == "ties":
        return rng.integers(-3, 4, size=(rows, cols)).astype(t)
    if kind == "full":
        v = rng.integers(info.min, info.max, size=(rows, cols), dtype=t, endpoint=True)
        ext = rng.random((rows, cols)) < 0.01
        v[ext] = np.where(rng.random(int(ext.sum())) < 0.5, info.min, info.max).astype(t)
        return v
    if kind == "constant":
        return np.repeat(rng.integers(info.min, info.max, size=(rows, 1), dtype=t), cols, axis=1)
    raise KeyError(kind)


def config_workloads(which: str) -> list[Workload]:
    """The workload(s) of one named configuration, at full size."""
    if which == "c1":
        return [c1_row32000_f32()]
    if which == "c2":
        return [c2_row202048_f32()]
    if which == "c3":
        return [c3_rows32_f16_bf16("f16"), c3_rows32_f16_bf16("bf16")]
    if which == "c4":
        return [c4_square_f32_f64("f32"), c4_square_f32_f64("f64")]
    if which == "c5a":
        return [c5a_many_rows_f32()]
    if which == "c5b":
        return [c5b_narrow_rows_f16()]
    if which == "axis":
        return [axis_many_outputs_f32(), axis_few_outputs_f32(), axis_element_loads_f16()]
    if which == "wide":
        return [wide_row_f16()]
    if which == "scan":
        return ([scan_doc_starts_i64()] + [scan_rows_i64(r, 65536 // r) for r in (1, 4, 64, 1024)]
                + [scan_row_65536(d) for d in ("i32", "f32", "f64")]
                + [scan_long_row_f32(), scan_many_rows_f32()])
    raise KeyError(which)


CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5a", "c5b")

# ----------------------------------------------------------------------------------------
# Generic generators for parity sweeps and fuzzing.

# Special values per format, as float64, all exactly representable in that format.
_MIN_SUBNORMAL = {"f32": 2.0 ** -149, "f16": 2.0 ** -24, "bf16": 2.0 ** -133, "f64": 2.0 ** -1074}
_MAX_FINITE = {"f32": float(np.finfo(np.float32).max), "f16": 65504.0,
               "bf16": float.fromhex("0x1.fep127"), "f64": float(np.finfo(np.float64).max)}


def special_alphabet(dtype: str) -> np.ndarray:
    """{NaN, -inf, -max, -1, -min_subnormal, -0, +0, +min_subnormal, 1, max, +inf} as float64."""
    s, m = _MIN_SUBNORMAL[dtype], _MAX_FINITE[dtype]
    return np.array([math.nan, -math.inf, -m, -1.0, -s, -0.0, 0.0, s, 1.0, m, math.inf])


# Bit layout of each floating-point storage format's NaNs: (bits type, exponent field all
# ones, payload bits below the quiet bit, sign bit). The quiet bit is the payload's top bit.
NAN_LAYOUT = {"f16": (np.uint16, 0x7C00, 0x01FF, 0x8000),
              "bf16": (np.uint16, 0x7F80, 0x003F, 0x8000),
              "f32": (np.uint32, 0x7F800000, 0x003FFFFF, 0x80000000),
              "f64": (np.uint64, 0x7FF0000000000000, 0x0007FFFFFFFFFFFF, 0x8000000000000000)}


def random_bit_rows(rng: np.random.Generator, rows: int, cols: int, dtype: str) -> np.ndarray:
    """A (rows, cols) storage array of uniformly random bit patterns (every class of the
    format: subnormals, both zeros, quiet NaNs of any payload and sign), with about one
    entry in eight, and element 0 of every fourth row, replaced by a signalling NaN (quiet
    bit clear, a non-zero payload below it, either sign)."""
    bt, expo, payload, sign = NAN_LAYOUT[dtype]
    u = rng.integers(0, np.iinfo(bt).max, size=(rows, cols), dtype=bt, endpoint=True)
    snan = (bt(expo) | rng.integers(1, payload, size=(rows, cols), dtype=bt, endpoint=True)
            | (rng.integers(0, 2, size=(rows, cols), dtype=bt) * bt(sign)))
    mask = rng.random((rows, cols)) < 0.125
    mask[::4, 0] = True
    u = np.where(mask, snan, u).astype(bt)
    return np.ascontiguousarray(u if dtype == "bf16" else u.view(STORAGE[dtype]))


def random_rows(rng: np.random.Generator, rows: int, cols: int, dtype: str, kind: str) -> np.ndarray:
    """A (rows, cols) storage array of one of several value kinds.

    normal   iid N(0,1)
    ties     N(0,1) quantised to 16 levels
    special  iid draws from the special-value alphabet (NaN, +-inf, +-0, subnormals, ...)
    mixed    N(0,1) with ~1% of entries replaced by alphabet draws
    constant one N(0,1) draw per row, repeated
    bits     uniformly random bit patterns with signalling NaNs planted (random_bit_rows)
    """
    if kind == "bits":
        return random_bit_rows(rng, rows, cols, dtype)
    if kind == "normal":
        v = rng.standard_normal((rows, cols))
    elif kind == "ties":
        v = quantised_normal(rng, (rows, cols))
    elif kind == "special":
        alpha = special_alphabet(dtype)
        v = alpha[rng.integers(0, alpha.size, size=(rows, cols))]
    elif kind == "mixed":
        v = rng.standard_normal((rows, cols))
        alpha = special_alphabet(dtype)
        mask = rng.random((rows, cols)) < 0.01
        v[mask] = alpha[rng.integers(0, alpha.size, size=int(mask.sum()))]
    elif kind == "constant":
        v = np.repeat(rng.standard_normal((rows, 1)), cols, axis=1)
    else:
        raise KeyError(kind)
    return to_storage(v, dtype)
