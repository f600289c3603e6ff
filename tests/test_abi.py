"""The C ABI on the host: the library loads, exports every declared symbol, validates its
arguments before touching the GPU, and plans launches by the documented rules (CPU only:
no kernel is launched here; planning runs under a simulated device capacity)."""
import os
import re

import pytest

import argmin_reduction_wide_amd.binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "argreduce.h")
MI355X_THREADS = 256 * 2048
H200_THREADS = 132 * 2048
INT32_MAX = 2 ** 31 - 1
FAKE = 1 << 20  # an aligned, never-dereferenced address
ESIZE = {B.F32: 4, B.F16: 2, B.BF16: 2, B.F64: 8}


@pytest.fixture
def lib():
    h = B.lib()
    yield h
    B.argreduce_debug_set_capacity(0)
    B.argreduce_debug_force_path(B.PATH_AUTO)
    B.argreduce_debug_set_window(0)


@pytest.fixture
def mi355x(lib):
    assert B.argreduce_debug_set_capacity(MI355X_THREADS) == 0
    return lib


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(argreduce_\w+)\s*\(", text, re.M)))


def test_header_declares_what_the_binding_names():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_has_no_oracle_dependency():
    # the product library must not link, load or name the CPU oracle
    blob = open(B.LIB_PATH, "rb").read()
    assert b"oracle" not in blob


@pytest.mark.parametrize("rows,cols,dtype,op,code", [
    (-1, 10, B.F32, B.MAX, -1),
    (4, 0, B.F32, B.MAX, -1),
    (4, -3, B.F32, B.MAX, -1),
    (4, 10, 7, B.MAX, -2),
    (4, 10, -1, B.MAX, -2),
    (4, 10, B.F32, 4, -1),
    (4, 10, B.F32, -1, -1),
    (1 << 40, 1 << 30, B.F16, B.MAX, -1),  # rows * cols * element size beyond int64
])
def test_invalid_arguments_rejected_before_any_gpu_call(lib, rows, cols, dtype, op, code):
    assert B.argreduce_lastaxis(FAKE, dtype, rows, cols, op, FAKE, 0, 0, 0) == code


def test_null_and_misaligned_pointers(lib):
    assert B.argreduce_lastaxis(0, B.F32, 2, 8, B.MAX, FAKE, 0, 0, 0) == -1
    assert B.argreduce_lastaxis(FAKE, B.F32, 2, 8, B.MAX, 0, 0, 0, 0) == -1
    assert B.argreduce_lastaxis(FAKE + 2, B.F32, 2, 8, B.MAX, FAKE, 0, 0, 0) == -1
    assert B.argreduce_lastaxis(FAKE + 4, B.F64, 2, 8, B.MAX, FAKE, 0, 0, 0) == -1
    assert B.argreduce_lastaxis(FAKE, B.F32, 2, 8, B.MAX, FAKE + 4, 0, 0, 0) == -1


def test_noalloc_entry_point_checks_before_any_gpu_call(lib):
    """argreduce_lastaxis_noalloc validates like argreduce_lastaxis, and refuses a plan
    whose scratch exceeds the library-held array (ARGREDUCE_NOALLOC_SCRATCH_BYTES, as the
    header defines it) before touching the device."""
    text = open(HEADER).read()
    m = re.search(r"#define ARGREDUCE_NOALLOC_SCRATCH_BYTES \((\d+)u \* (\d+)u\)", text)
    assert m and int(m.group(1)) * int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
    f = lib.argreduce_lastaxis_noalloc
    assert f(FAKE, B.F32, -1, 10, B.MAX, FAKE, 0) == -1
    assert f(FAKE, B.F32, 4, 0, B.MAX, FAKE, 0) == -1
    assert f(FAKE, 9, 4, 10, B.MAX, FAKE, 0) == -2
    assert f(FAKE, B.F32, 4, 10, 7, FAKE, 0) == -1
    assert f(0, B.F32, 4, 10, B.MAX, FAKE, 0) == -1
    assert f(FAKE, B.F32, 4, 10, B.MAX, FAKE + 4, 0) == -1
    assert f(0, B.F32, 0, 10, B.MAX, 0, 0) == 0
    # the largest split scratch at MI355X capacity fits; a device four times larger does not
    B.argreduce_debug_set_capacity(MI355X_THREADS)
    assert B.argreduce_scratch_bytes(8, 1 << 20, B.F64) == 15 + 2048 * 32 <= B.NOALLOC_SCRATCH_BYTES
    B.argreduce_debug_set_capacity(4 * MI355X_THREADS)
    assert B.argreduce_scratch_bytes(32, 1 << 20, B.F64) > B.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, B.F64, 32, 1 << 20, B.MAX, FAKE, 0) == -4


def test_zero_rows_is_a_no_op(lib):
    assert B.argreduce_lastaxis(0, B.F32, 0, 8, B.MAX, 0, 0, 0, 0) == 0


def test_scratch_too_small_is_detected_before_launch(mi355x):
    need = B.argreduce_scratch_bytes(1, 202048, B.F32)
    assert 0 < need < 64 * 1024
    assert B.argreduce_lastaxis(FAKE, B.F32, 1, 202048, B.MAX, FAKE, FAKE, need - 1, 0) == -4
    assert B.argreduce_lastaxis(FAKE, B.F32, 1, 202048, B.MAX, FAKE, 0, need, 0) == -4


def test_scratch_bytes_invalid_arguments(lib):
    assert B.argreduce_scratch_bytes(1, 0, B.F32) == B.SIZE_MAX
    assert B.argreduce_scratch_bytes(-1, 5, B.F32) == B.SIZE_MAX
    assert B.argreduce_scratch_bytes(1 << 40, 1 << 30, B.F32) == B.SIZE_MAX
    assert B.argreduce_scratch_bytes(1, 5, 9) == B.SIZE_MAX


@pytest.mark.parametrize("dtype", [B.F32, B.F16, B.BF16, B.F64])
@pytest.mark.parametrize("cap", [MI355X_THREADS, H200_THREADS, 4096])
def test_scratch_is_bounded_by_device_capacity(lib, dtype, cap):
    """Scratch stays in the low kilobytes for any shape, INT_MAX widths included."""
    B.argreduce_debug_set_capacity(cap)
    # a split row's workgroups publish 2 (f64: 4) 8-byte words each, and one device wave
    # of workgroups bounds how many there are
    entry = 32 if dtype == B.F64 else 16
    bound = 15 + entry * (cap // 256)
    for rows in (1, 2, 7, 32, 1000, cap // 256 - 1, cap // 256, 65536):
        for cols in (1, 63, 64, 4096, 202048, 2 ** 24, INT32_MAX):
            s = B.argreduce_scratch_bytes(rows, cols, dtype)
            assert s != B.SIZE_MAX and s <= bound, (rows, cols, s, bound)


def test_plan_paths_for_the_measured_shapes(mi355x):
    p = B.argreduce_plan(1, 202048, B.F32)
    assert p["path"] == B.PATH_SPLIT and p["blocks_per_row"] > 1
    assert p["scratch_bytes"] == B.argreduce_scratch_bytes(1, 202048, B.F32)
    assert B.argreduce_plan(32, 202048, B.F16)["path"] == B.PATH_SPLIT
    assert B.argreduce_plan(1, 32000, B.F32)["path"] == B.PATH_SPLIT
    p = B.argreduce_plan(65536, 64, B.F16)
    assert p["path"] == B.PATH_SUBWAVE and p["lanes_per_row"] == 8
    assert B.argreduce_plan(65536, 1024, B.F32)["lanes_per_row"] == 64
    p = B.argreduce_plan(4096, 4096, B.F32)  # 16 KiB rows: a workgroup each, one step
    assert p["path"] == B.PATH_BLOCK and p["unroll"] == 4 and p["grid_blocks"] == 4096
    p = B.argreduce_plan(4096, 4096, B.F64)
    assert p["path"] == B.PATH_BLOCK and p["unroll"] == 8
    assert B.argreduce_plan(4096, 8, B.F32)["lanes_per_row"] == 2


def split_rule(rows, vec, cap_blocks):
    """(B, U) of the split plan's rule, written out: the fewest U <= 4 with B =
    ceil(vec / (256 U)) <= 65 and rows * B within a device wave; else the fewest U <= 8 with
    B <= 256 and the same bound; else None (several steps)."""
    for max_b, us in ((65, (1, 2, 4)), (256, (1, 2, 4, 8))):
        for u in us:
            b = -(-vec // (256 * u))
            if b <= max_b and rows * b <= cap_blocks:
                return b, u
    return None


def test_plan_keeps_every_lane_busy_and_one_device_wave(mi355x):
    """Split rows take the fewest 16-byte loads per lane (U) for which one step of
    ceil(vectors / (256 U)) workgroups per row covers the row with all rows' workgroups in
    one device wave (so no workgroup is idle): first at most 65 workgroups per row with
    U <= 4 (one candidate per lane of the finalizer's first wavefront), then at most 256
    with U <= 8; else 8 loads per lane and several steps."""
    cap_blocks = MI355X_THREADS // 256
    seen = set()
    for rows, cols, dtype in [(1, 32000, B.F32), (1, 202048, B.F32), (8, 202048, B.F32),
                              (32, 202048, B.F16), (64, 202048, B.BF16), (1, 2 ** 24, B.F64),
                              (100, 50000, B.BF16), (300, 40000, B.F32), (256, 202048, B.F16),
                              (1, 1 << 20, B.F32), (1, 1 << 21, B.F32), (1, 500000, B.F32),
                              (8, 65536, B.F32), (32, 65536, B.F32)]:
        p = B.argreduce_plan(rows, cols, dtype)
        assert p["path"] == B.PATH_SPLIT, (rows, cols, p)
        esize = {B.F32: 4, B.F16: 2, B.BF16: 2, B.F64: 8}[dtype]
        vec = -(-cols * esize // 16)
        b, u = p["blocks_per_row"], p["unroll"]
        assert p["grid_blocks"] == rows * b <= cap_blocks and p["grid_rows"] == rows
        want = split_rule(rows, vec, cap_blocks)
        if want:
            assert (b, u) == want, (rows, cols, p)
            assert b * 256 * u >= vec > (b - 1) * 256 * u  # one step, no idle workgroup
            seen.add("wave" if b <= 65 else "block")
        else:
            assert u == 8 and b == cap_blocks // 4 // rows  # several steps of 8 loads
            seen.add("steps")
    assert seen == {"wave", "block", "steps"}
    assert (B.argreduce_plan(1, 202048, B.F32)["blocks_per_row"],
            B.argreduce_plan(1, 202048, B.F32)["unroll"]) == (50, 4)
    assert (B.argreduce_plan(32, 202048, B.F16)["blocks_per_row"],
            B.argreduce_plan(32, 202048, B.F16)["unroll"]) == (50, 2)


def test_split_is_bounded_by_capacity(lib):
    """At an H200-sized capacity (1056 workgroups of 256 threads) [1, 202048] fp32 takes four
    vectors per lane (50 workgroups), and [32, 202048] fp32 needs 8 per lane for its 32 rows
    to fit: 25 workgroups per row, 800 in all. [8, 202048] fp32 takes 4 per lane at MI355X
    capacity (400 workgroups) but 8 at an eight-times smaller one (256 workgroups)."""
    B.argreduce_debug_set_capacity(H200_THREADS)
    p = B.argreduce_plan(1, 202048, B.F32)
    assert p["path"] == B.PATH_SPLIT and p["blocks_per_row"] == 50 and p["unroll"] == 4
    p = B.argreduce_plan(32, 202048, B.F32)
    assert p["path"] == B.PATH_SPLIT and p["blocks_per_row"] == 25 and p["unroll"] == 8
    assert p["grid_blocks"] == 800 <= H200_THREADS // 256
    B.argreduce_debug_set_capacity(MI355X_THREADS)
    assert B.argreduce_plan(8, 202048, B.F32)["unroll"] == 4
    B.argreduce_debug_set_capacity(MI355X_THREADS // 8)
    p = B.argreduce_plan(8, 202048, B.F32)
    assert p["unroll"] == 8 and p["grid_blocks"] == 200
    p = B.argreduce_plan(512, 202048, B.F32)  # no one-step split fits: a quarter device wave
    assert p["path"] == B.PATH_BLOCK and p["unroll"] == 8


def test_narrow_groups_take_at_most_one_device_wave(mi355x):
    """Groups narrower than a wavefront on rows of whole 16-byte vectors, or on rows whose
    span of vectors (from the one holding the row's first byte, in a 16-byte aligned tensor)
    the group covers, launch at most one device wave of workgroups (2048 on MI355X) and loop
    over rows; other rows, and a wavefront per row, keep a workgroup per 256 / G rows.
    [65536,250] bf16: 500-byte rows from offsets up to 12, 32 vectors for 32 lanes;
    [300000,10] fp32: 3 of 4; [100000,63] fp16: 9 for 8; [300000,7] fp32: 3 for 2."""
    cases = [((65536, 100, B.F32), 32, 2048), ((200000, 40, B.F32), 16, 2048),
             ((65536, 64, B.F16), 8, 2048), ((1 << 21, 4, B.F32), 1, 2048),
             ((40000, 64, B.F16), 8, 1250), ((65536, 250, B.BF16), 32, 2048),
             ((300000, 10, B.F32), 4, 2048), ((100000, 63, B.F16), 8, 3125),
             ((300000, 7, B.F32), 2, 2344), ((65536, 1024, B.F32), 64, 16384)]
    for (rows, cols, dtype), lanes, grid in cases:
        p = B.argreduce_plan(rows, cols, dtype)
        assert p["path"] == B.PATH_SUBWAVE and p["lanes_per_row"] == lanes, (rows, cols, p)
        assert p["grid_blocks"] == grid, (rows, cols, p)
        assert p["grid_rows"] == grid * (256 // lanes)


def test_small_capacity_forces_row_loops(lib):
    B.argreduce_debug_set_capacity(1024)  # four workgroups; grids hold 64 device-fulls
    p = B.argreduce_plan(1000, 100000, B.F32)
    assert p["path"] == B.PATH_BLOCK and p["grid_rows"] < 1000 and p["grid_blocks"] <= 4 * 64
    p = B.argreduce_plan(100000, 64, B.F32)
    assert p["grid_rows"] < 100000 and p["grid_blocks"] <= 4 * 64


def test_forced_paths(mi355x):
    assert B.argreduce_debug_force_path(B.PATH_SPLIT) == 0
    p = B.argreduce_plan(3, 7, B.F32)
    assert p["path"] == B.PATH_SPLIT and p["blocks_per_row"] >= 2 and p["scratch_bytes"] > 0
    assert B.argreduce_debug_force_path(B.PATH_BLOCK) == 0
    p = B.argreduce_plan(1, 202048, B.F32)
    assert p["path"] == B.PATH_BLOCK and p["blocks_per_row"] == 1 and p["scratch_bytes"] == 0
    assert B.argreduce_debug_force_path(B.PATH_SUBWAVE) == 0
    p = B.argreduce_plan(1, 202048, B.F32)
    assert p["path"] == B.PATH_SUBWAVE and p["lanes_per_row"] == 64
    # one lane per row (the serial "before" kernel): a one-lane group, one load in flight,
    # 256 rows per workgroup; never chosen without the override
    assert B.argreduce_debug_force_path(B.PATH_THREAD) == 0
    for rows, cols, dtype in [(1, 202048, B.F32), (32, 202048, B.F16), (700, 129, B.F64), (1, 1, B.F32)]:
        p = B.argreduce_plan(rows, cols, dtype)
        assert (p["path"], p["lanes_per_row"], p["unroll"], p["scratch_bytes"]) == (B.PATH_SUBWAVE, 1, 1, 0), p
        assert p["grid_blocks"] == -(-rows // 256)
    assert B.argreduce_debug_force_path(7) == -1 and B.argreduce_debug_force_path(B.PATH_AXIS) == -1
    assert B.argreduce_debug_set_capacity(-5) == -1


@pytest.mark.parametrize("outer,length,inner,dtype,code", [
    (-1, 10, 4, B.F32, -1), (2, 0, 4, B.F32, -1), (2, 10, 0, B.F32, -1),
    (2, 10, 4, 9, -2), (1, INT32_MAX + 1, 2, B.F16, -3),
])
def test_axis_invalid_arguments(lib, outer, length, inner, dtype, code):
    assert B.argreduce_axis(FAKE, dtype, outer, length, inner, B.MAX, FAKE, 0, 0, 0) == code


def test_axis_zero_outer_and_op_check(lib):
    assert B.argreduce_axis(0, B.F32, 0, 10, 4, B.MAX, 0, 0, 0, 0) == 0
    assert B.argreduce_axis(FAKE, B.F32, 2, 10, 4, 7, FAKE, 0, 0, 0) == -1


def test_axis_plans(mi355x):
    # inner == 1 is the last-axis reduction, with its plan and scratch
    assert B.argreduce_axis_plan(1, 202048, 1, B.F32) == B.argreduce_plan(1, 202048, B.F32)
    assert B.argreduce_axis_scratch_bytes(1, 202048, 1, B.F32) == B.argreduce_scratch_bytes(1, 202048, B.F32)
    p = B.argreduce_axis_plan(4096, 512, 256, B.F32)  # more tiles than resident workgroups
    assert p["path"] == B.PATH_AXIS and p["blocks_per_row"] == 1 and p["scratch_bytes"] == 0
    assert p["outputs_per_block"] == 256 and p["load_bytes"] == 16 and p["dispatches"] == 1
    p = B.argreduce_axis_plan(1, 1 << 20, 32, B.F32)  # few outputs, long axis: split
    assert p["path"] == B.PATH_AXIS and p["blocks_per_row"] > 1 and p["dispatches"] == 2
    assert p["scratch_bytes"] == 15 + p["blocks_per_row"] * 32 * 8
    assert p["grid_blocks"] <= MI355X_THREADS // 256
    # split width: a quarter of the device wave of workgroups (512 for one tile), or up to 1.5
    # times that when it covers the axis in one step per thread (1024 rows of 8 fp32 each)
    assert B.argreduce_axis_plan(1, 600000, 8, B.F32)["blocks_per_row"] == 586
    assert B.argreduce_axis_plan(1, 786432, 8, B.F32)["blocks_per_row"] == 768
    assert B.argreduce_axis_plan(1, 786433, 8, B.F32)["blocks_per_row"] == 512
    assert B.argreduce_axis_plan(1, 1000000, 8, B.F32)["blocks_per_row"] == 512
    # lanes: the next power of two of the vectors (16-byte loads) or elements per inner row
    for (inner, dtype), (tile, load) in {
        (3, B.F16): (4, 2), (9, B.F16): (16, 2), (16, B.F16): (16, 16), (8, B.BF16): (8, 16),
        (6, B.F64): (8, 16), (4, B.F32): (4, 16), (260, B.F32): (256, 16), (250, B.F32): (64, 4),
        (2, B.F32): (2, 4), (1000, B.F64): (128, 16),
    }.items():
        p = B.argreduce_axis_plan(3, 100, inner, dtype)
        assert (p["outputs_per_block"], p["load_bytes"]) == (tile, load), (inner, dtype, p)
        # positions per thread and step: 8 with 16-byte loads (4 for fp64); element loads keep
        # 64 bytes in flight per lane
        want_u = (4 if dtype == B.F64 else 8) if load == 16 else 64 // ESIZE[dtype]
        assert p["unroll"] == want_u, (inner, dtype, p)
        lanes = tile // (16 // ESIZE[dtype] if load == 16 else 1)  # lanes along inner
        assert p["lanes_per_row"] == p["blocks_per_row"] * (256 // lanes)  # threads per output


def test_axis_two_workgroups_per_tile(mi355x):
    """Where a quarter of a device wave gives two workgroups per tile (256 tiles), 16-byte
    loads take one per tile (no merge dispatch) and element loads keep two."""
    p = B.argreduce_axis_plan(256, 1024, 256, B.F32)
    assert (p["load_bytes"], p["blocks_per_row"], p["dispatches"]) == (16, 1, 1), p
    p = B.argreduce_axis_plan(64, 4096, 255, B.F32)
    assert (p["load_bytes"], p["blocks_per_row"], p["dispatches"]) == (4, 2, 2), p


def test_axis_plans_with_more_tiles_than_a_quarter_wave(mi355x):
    """Element-load plans (x off a 16-byte boundary, as the scratch query also sizes for)
    whose tiles outnumber a quarter of a device wave of workgroups: one workgroup per tile,
    a grid of at least one workgroup, and a scratch query that returns (a zero split here
    once divided the grid size by zero on the host)."""
    import itertools

    for outer, length, inner in itertools.product([1, 64, 256, 5000, 70000], [1, 16, 1000, 65536],
                                                  [2, 33, 63, 256, 1001]):
        if outer * length * inner > (1 << 34):
            continue
        for dtype in (B.F32, B.F16, B.BF16, B.F64):
            need = B.argreduce_axis_scratch_bytes(outer, length, inner, dtype)
            assert need < (1 << 40), (outer, length, inner, dtype, need)
            p = B.argreduce_axis_plan(outer, length, inner, dtype)
            assert p["blocks_per_row"] >= 1 and p["grid_blocks"] >= 1, (outer, length, inner, p)
    assert B.argreduce_axis_scratch_bytes(256, 16, 256, B.F16) == 0


def test_forced_split_geometry(mi355x):
    """argreduce_debug_force_split: every last-axis plan becomes a split of the given
    workgroups per row and loads per lane (several steps when one does not cover the row),
    invalid values are refused, and 0 restores the automatic plans."""
    auto = B.argreduce_plan(32, 202048, B.F16)
    try:
        assert B.argreduce_debug_force_split(8, 4) == 0
        for rows, cols in ((32, 202048), (1, 1000), (4096, 4096)):
            p = B.argreduce_plan(rows, cols, B.F16)
            assert (p["path"], p["blocks_per_row"], p["unroll"]) == (B.PATH_SPLIT, 8, 4), p
            assert p["grid_blocks"] == rows * 8
            assert B.argreduce_scratch_bytes(rows, cols, B.F16) >= rows * 8 * 16
        for b, u in ((1, 4), (2048, 4), (8, 3), (8, 16), (-1, 1)):
            assert B.argreduce_debug_force_split(b, u) == -1, (b, u)  # ARGREDUCE_ERR_INVALID_ARG
    finally:
        assert B.argreduce_debug_force_split(0) == 0
    assert B.argreduce_plan(32, 202048, B.F16) == auto


def test_axis_forced_paths(mi355x):
    B.argreduce_debug_force_path(B.PATH_SPLIT)
    assert B.argreduce_axis_plan(64, 100, 256, B.F32)["blocks_per_row"] >= 2
    B.argreduce_debug_force_path(B.PATH_BLOCK)
    assert B.argreduce_axis_plan(1, 1 << 20, 32, B.F32)["blocks_per_row"] == 1


def test_axis_scratch_too_small(mi355x):
    need = B.argreduce_axis_scratch_bytes(1, 1 << 20, 32, B.F32)
    assert 0 < need < (1 << 20)
    # FAKE is 16-byte aligned: the call takes the aligned plan
    aligned = B.argreduce_axis_plan(1, 1 << 20, 32, B.F32)["scratch_bytes"]
    assert 0 < aligned <= need
    assert B.argreduce_axis(FAKE, B.F32, 1, 1 << 20, 32, B.MAX, FAKE, FAKE, aligned - 1, 0) == -4


# cumulative scan (cummax / cummin)


@pytest.mark.parametrize("dtype,rows,cols,op,code", [
    (9, 2, 8, B.MAX, -2), (B.F32, 2, 8, B.MAX_LAST, -1), (B.F32, 2, 8, 7, -1),
    (B.F32, 2, 0, B.MAX, -1), (B.F32, -1, 8, B.MAX, -1), (B.I64, 1, INT32_MAX + 1, B.MAX, -3),
])
def test_scan_invalid_arguments(lib, dtype, rows, cols, op, code):
    assert B.argreduce_scan_lastaxis(FAKE, dtype, rows, cols, op, FAKE * 4, FAKE * 8, 0, 0, 0) == code


def test_scan_pointer_checks(lib):
    x, v, i = FAKE, FAKE * 4, FAKE * 8
    assert B.argreduce_scan_lastaxis(0, B.F32, 0, 8, B.MAX, 0, 0, 0, 0, 0) == 0  # no rows
    assert B.argreduce_scan_lastaxis(0, B.F32, 2, 8, B.MAX, v, i, 0, 0, 0) == -1
    assert B.argreduce_scan_lastaxis(x, B.F32, 2, 8, B.MAX, 0, i, 0, 0, 0) == -1
    assert B.argreduce_scan_lastaxis(x, B.F32, 2, 8, B.MAX, v, 0, 0, 0, 0) == -1
    assert B.argreduce_scan_lastaxis(x + 2, B.F32, 2, 8, B.MAX, v, i, 0, 0, 0) == -1
    assert B.argreduce_scan_lastaxis(x, B.I64, 2, 8, B.MAX, v + 4, i, 0, 0, 0) == -1
    assert B.argreduce_scan_lastaxis(x, B.F32, 2, 8, B.MAX, v, i + 4, 0, 0, 0) == -1
    # outputs overlapping the input or each other
    assert B.argreduce_scan_lastaxis(x, B.F32, 2, 8, B.MAX, x + 32, i, 0, 0, 0) == -1
    assert B.argreduce_scan_lastaxis(x, B.F32, 2, 8, B.MAX, v, x + 8, 0, 0, 0) == -1
    assert B.argreduce_scan_lastaxis(x, B.F32, 2, 8, B.MAX, v, v + 16, 0, 0, 0) == -1


def test_other_entry_points_refuse_integers(lib):
    for dt in (B.I32, B.I64):
        assert B.argreduce_lastaxis(FAKE, dt, 2, 8, B.MAX, FAKE, 0, 0, 0) == -2
        assert B.argreduce_axis(FAKE, dt, 2, 8, 3, B.MAX, FAKE, 0, 0, 0) == -2
        assert B.argreduce_scratch_bytes(2, 8, dt) == B.SIZE_MAX


def test_scan_plans_and_scratch(mi355x):
    # tiles: 256 lanes x U chunks of 16 bytes. A row that fits one tile of U <= 2 takes the
    # smallest such tile; else U = 1 while a row needs <= 64 tiles and the grid stays within
    # two device waves, else U = 2 within 64 tiles; longer rows the smallest of U = 2, 4, 8
    # whose grid is at most a quarter of a device wave (512 workgroups), else U = 8.
    p = B.argreduce_scan_plan(1, 65536, B.I64)  # 128 tiles of U = 1: U = 2
    assert p["path"] == B.PATH_SCAN and p["unroll"] == 2 and p["outputs_per_block"] == 1024
    assert p["blocks_per_row"] == 64 and p["grid_blocks"] == 64 and p["load_bytes"] == 16
    assert p["scratch_bytes"] == 15 + 64 * 2 * 4 * 8  # aggregate + prefix, 4 words each
    assert B.argreduce_scan_scratch_bytes(1, 65536, B.I64) == p["scratch_bytes"]
    p = B.argreduce_scan_plan(1, 65536, B.F32)  # 64 tiles of U = 1
    assert p["unroll"] == 1 and p["outputs_per_block"] == 1024 and p["blocks_per_row"] == 64
    p = B.argreduce_scan_plan(4096, 1024, B.F32)  # one U = 1 tile per row: no look-back
    assert p["unroll"] == 1 and p["blocks_per_row"] == 1 and p["scratch_bytes"] == 0
    p = B.argreduce_scan_plan(64, 1024, B.I64)  # one U = 2 tile rather than two U = 1 tiles
    assert p["unroll"] == 2 and p["blocks_per_row"] == 1 and p["scratch_bytes"] == 0
    p = B.argreduce_scan_plan(4096, 4096, B.F32)  # U = 1 would make 16384 workgroups
    assert p["unroll"] == 2 and p["outputs_per_block"] == 2048
    assert p["blocks_per_row"] == 2 and p["grid_blocks"] == 8192
    assert p["scratch_bytes"] == B.argreduce_scan_scratch_bytes(4096, 4096, B.F32) > 0
    p = B.argreduce_scan_plan(3, 8193, B.F16)
    assert p["unroll"] == 1 and p["outputs_per_block"] == 2048 and p["blocks_per_row"] == 5
    assert p["load_bytes"] == 2 and p["scratch_bytes"] == 15 + 3 * 5 * 2 * 2 * 8
    p = B.argreduce_scan_plan(1, 64 * 4096 + 1, B.F32)  # 129 tiles of U = 2
    assert p["unroll"] == 2 and p["outputs_per_block"] == 2048 and p["blocks_per_row"] == 129
    assert B.argreduce_scan_plan(1, 64 * 2048, B.F32)["unroll"] == 2
    assert B.argreduce_scan_plan(1, 64 * 2048 + 1, B.F32)["unroll"] == 2
    for rows, cols, dtype, u in [(1, 1 << 20, B.F32, 2), (1, 512 * 2048 + 1, B.F32, 4),
                                 (1, 1 << 21, B.F32, 4), (1, 1 << 22, B.F32, 8),
                                 (8, 1 << 18, B.F32, 4), (4, 1 << 18, B.F32, 2),
                                 (16, 1 << 18, B.F32, 8), (1, 1 << 21, B.F16, 2),
                                 (1, 1 << 20, B.I64, 4), (1, 1 << 22, B.I64, 8)]:
        p = B.argreduce_scan_plan(rows, cols, dtype)
        assert p["unroll"] == u, (rows, cols, dtype, p)
        assert u == 8 or p["grid_blocks"] <= 512
    assert B.argreduce_scan_plan(2, 1 << 24, B.F32)["blocks_per_row"] == 2048
    assert B.argreduce_scan_scratch_bytes(2, 0, B.F32) == B.SIZE_MAX
    assert B.argreduce_scan_scratch_bytes(2, 8, 9) == B.SIZE_MAX


def test_scan_scratch_too_small(mi355x):
    need = B.argreduce_scan_scratch_bytes(1, 65536, B.I64)
    assert B.argreduce_scan_lastaxis(FAKE, B.I64, 1, 65536, B.MAX, FAKE * 4, FAKE * 8, FAKE,
                                     need - 1, 0) == -4
    assert B.argreduce_scan_lastaxis(FAKE, B.I64, 1, 65536, B.MAX, FAKE * 4, FAKE * 8, 0,
                                     need, 0) == -4


# rows wider than INT32_MAX: windows


def test_wide_rows_plan(mi355x):
    p = B.argreduce_plan(1, INT32_MAX + 1, B.F16)
    assert p["path"] == B.PATH_WIDE and p["dispatches"] == 2
    w = p["window"]
    assert 0 < w <= 1 << 30 and w % 4096 == 0
    assert p["blocks_per_row"] == -(-(INT32_MAX + 1) // w) and p["grid_blocks"] == p["blocks_per_row"]
    assert p["blocks_per_row"] >= MI355X_THREADS // 256  # about one window per resident workgroup
    assert p["scratch_bytes"] == 15 + p["blocks_per_row"] * 16
    assert B.argreduce_scratch_bytes(1, INT32_MAX + 1, B.F16) == p["scratch_bytes"]
    p = B.argreduce_plan(3, 5 * 2 ** 31, B.F64)
    assert p["path"] == B.PATH_WIDE and p["window"] <= 1 << 30 and p["grid_blocks"] == 3 * p["blocks_per_row"]
    assert p["scratch_bytes"] == 15 + 3 * p["blocks_per_row"] * 16
    # the last ordinary width keeps its path
    assert B.argreduce_plan(1, INT32_MAX, B.F16)["path"] == B.PATH_SPLIT
    # wide rows are refused by the middle-axis and scan entry points only
    assert B.argreduce_axis(FAKE, B.F32, 2, INT32_MAX + 1, 3, B.MAX, FAKE, 0, 0, 0) == -3
    assert B.argreduce_scan_lastaxis(FAKE, B.F32, 1, INT32_MAX + 1, B.MAX, FAKE * 4, FAKE * 8,
                                     0, 0, 0) == -3
    assert B.argreduce_lastaxis(FAKE, B.F16, 1, INT32_MAX + 1, B.MAX, FAKE, FAKE, 100, 0) == -4


def test_forced_window(mi355x):
    assert B.argreduce_debug_set_window(-1) == -1 and B.argreduce_debug_set_window((1 << 30) + 1) == -1
    assert B.argreduce_debug_force_path(B.PATH_AXIS) == -1 and B.argreduce_debug_force_path(B.PATH_SCAN) == -1
    assert B.argreduce_debug_force_path(B.PATH_WIDE) == 0
    assert B.argreduce_debug_set_window(1000) == 0
    p = B.argreduce_plan(5, 2500, B.F32)
    assert p["path"] == B.PATH_WIDE and p["window"] == 1000 and p["blocks_per_row"] == 3
    assert p["grid_blocks"] == 15 and p["unroll"] == 2 and p["scratch_bytes"] == 15 + 15 * 16
    B.argreduce_debug_set_window(0)
    p = B.argreduce_plan(1, 202048, B.F32)  # forced, automatic window
    assert p["path"] == B.PATH_WIDE and p["window"] == 4096


def test_debug_hooks_validate(lib):
    assert B.argreduce_debug_launch_store(0, 0) == -1
    assert B.argreduce_debug_launch_store(FAKE + 4, 0) == -1
    # the streaming-read hook: null, unaligned, ragged or empty sizes, grid out of range
    assert B.argreduce_debug_launch_read(0, 4096, FAKE, 1, 0) == -1
    assert B.argreduce_debug_launch_read(FAKE, 4096, 0, 1, 0) == -1
    assert B.argreduce_debug_launch_read(FAKE + 8, 4096, FAKE, 1, 0) == -1
    assert B.argreduce_debug_launch_read(FAKE, 4100, FAKE, 1, 0) == -1
    assert B.argreduce_debug_launch_read(FAKE, 0, FAKE, 1, 0) == -1
    assert B.argreduce_debug_launch_read(FAKE, 4096, FAKE + 2, 1, 0) == -1
    assert B.argreduce_debug_launch_read(FAKE, 4096, FAKE, 0, 0) == -1
    assert B.argreduce_debug_launch_read(FAKE, 4096, FAKE, 65537, 0) == -1
    assert B.argreduce_debug_set_spin_limit(0) == 0
