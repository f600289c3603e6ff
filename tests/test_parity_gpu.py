"""GPU parity: the HIP library against the CPU oracle, bit for bit (int64 indices).

Covers the six measured workloads at full size, the pages' axis-length sweep and our own
dispatch thresholds, every launch path forced on ragged and misaligned rows under several
simulated device capacities, a special-value fuzz, widths straddling the widest scan step,
scratch handling (offsets, dirty contents, undersized buffers), HIP graph capture and
replay, and INT32_MAX-wide rows. Each case is printed before it runs.
"""
import numpy as np
import pytest

import argmin_reduction_wide_amd.binding as B
from argmin_reduction_wide_amd import workloads as W
from gpu_helpers import announce, check, run, to_device

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16", "f64")
OPS = ("max", "min", "max_last", "min_last")
VW = {"f32": 4, "f16": 8, "bf16": 8, "f64": 2}
H200_THREADS = 132 * 2048


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU; none is visible"
    B.argreduce_debug_set_capacity(0)
    B.argreduce_debug_force_path(B.PATH_AUTO)
    yield
    B.argreduce_debug_set_capacity(0)
    B.argreduce_debug_force_path(B.PATH_AUTO)


@pytest.fixture
def hooks():
    yield
    B.argreduce_debug_set_capacity(0)
    B.argreduce_debug_force_path(B.PATH_AUTO)


def test_device_plan_is_sane():
    p = B.argreduce_plan(1, 202048, "f32")
    announce(f"plan [1,202048] f32 on this device: {p}")
    assert p["device_threads"] >= 256 * 64
    assert p["path"] == B.PATH_SPLIT


@pytest.mark.parametrize("which", W.CONFIG_NAMES)
def test_config_full_size(oracle_lib, which):
    for w in W.config_workloads(which):
        for op in w.ops:
            got = check(oracle_lib, w.data, w.dtype, op, f"config {which} {w.name} plan="
                        f"{B.argreduce_plan(w.rows, w.cols, w.dtype)}")
            for row, want in w.planted.get(op, {}).items():
                assert got[row] == want, (w.name, op, row)


@pytest.mark.parametrize("which", W.CONFIG_NAMES)
def test_config_full_size_last_index(oracle_lib, which):
    """The same workloads under the last-index ops (ties to the highest index)."""
    for w in W.config_workloads(which):
        for op in w.ops:
            check(oracle_lib, w.data, w.dtype, op + "_last", f"config {which} {w.name} last")


def sweep_cols(dtype):
    v = VW[dtype]
    base = [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
            300, 1000, 1023, 1025, 4095, 4097, 129280]
    # our thresholds: 32 vectors (group -> wavefront), 256 (wavefront -> workgroup) and
    # 2048 (workgroup -> split)
    for nvec in (32, 256, 2048):
        base += [nvec * v - 1, nvec * v, nvec * v + 1]
    return sorted(set(base))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_axis_length_sweep(oracle_lib, dtype, op):
    """Axis lengths of both sides of every threshold x rows 1 / 3 / 300 x value kinds."""
    rng = np.random.default_rng(100 + DTYPES.index(dtype) * 2 + OPS.index(op))
    for cols in sweep_cols(dtype):
        for rows in (1, 3, 300):
            if rows * cols > 8_000_000:
                continue
            for kind in ("normal", "ties", "constant", "mixed", "bits"):
                arr = W.random_rows(rng, rows, cols, dtype, kind)
                check(oracle_lib, arr, dtype, op, f"sweep cols={cols} rows={rows} kind={kind}")


FORCED_SHAPES = [(1, 1), (1, 5), (2, 17), (5, 300), (33, 1000), (3, 40000), (700, 129), (4, 70001)]


@pytest.mark.parametrize("path", [B.PATH_SUBWAVE, B.PATH_BLOCK, B.PATH_SPLIT, B.PATH_THREAD])
@pytest.mark.parametrize("cap", [0, 1024, H200_THREADS])
def test_forced_paths_ragged_misaligned(oracle_lib, hooks, path, cap):
    rng = np.random.default_rng(7 + path * 10 + cap % 97)
    B.argreduce_debug_set_capacity(cap)
    B.argreduce_debug_force_path(path)
    for dtype in DTYPES:
        for rows, cols in FORCED_SHAPES:
            for offset in (0, 1, 3):
                arr = W.random_rows(rng, rows, cols, dtype, "mixed" if offset else "ties")
                for op in OPS:
                    check(oracle_lib, arr, dtype, op,
                          f"forced path={path} cap={cap} offset={offset} "
                          f"plan={B.argreduce_plan(rows, cols, dtype)}", offset_elems=offset)


@pytest.mark.parametrize("dtype", DTYPES)
def test_narrow_aligned_rows(oracle_lib, hooks, dtype):
    """Rows of 1..32 whole 16-byte vectors starting 16-byte aligned (the narrow kernel: a
    group of G = next power of two lanes per row, lanes past the row masked, position 0 from
    lane 0's own vector): every vector count around the powers of two, special values with a
    leading NaN in some rows, every op; then, under a four-workgroup capacity, more rows
    than the grid holds (groups loop over rows); and the same widths one element short
    (misaligned: the generic lane-group kernel) for contrast."""
    rng = np.random.default_rng(1300 + DTYPES.index(dtype))
    v = VW[dtype]
    for nvec in (1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 17, 24, 31, 32):
        cols = nvec * v
        for rows in (1, 7, 300):
            for kind in ("special", "ties", "mixed", "bits"):
                arr = W.random_rows(rng, rows, cols, dtype, kind)
                if kind == "special":
                    arr[::3, 0] = W.to_storage(np.array([np.nan]), dtype)[0]
                for op in OPS:
                    check(oracle_lib, arr, dtype, op, f"narrow nvec={nvec} rows={rows} kind={kind} "
                          f"plan={B.argreduce_plan(rows, cols, dtype)}")
        if cols > 1:
            arr = W.random_rows(rng, 5, cols - 1, dtype, "ties")
            check(oracle_lib, arr, dtype, "max", f"narrow-minus-one cols={cols - 1}")
    B.argreduce_debug_set_capacity(1024)
    for nvec in (3, 8, 32):
        arr = W.random_rows(rng, 20000, nvec * v, dtype, "ties")
        p = B.argreduce_plan(20000, nvec * v, dtype)
        assert p["grid_rows"] < 20000, p
        for op in OPS:
            check(oracle_lib, arr, dtype, op, f"narrow row loop nvec={nvec} plan={p}")


@pytest.mark.parametrize("path", [B.PATH_BLOCK, B.PATH_SPLIT])
@pytest.mark.parametrize("dtype", DTYPES)
def test_aligned_one_step_rows(oracle_lib, hooks, path, dtype):
    """Rows of whole 16-byte vectors from a 16-byte aligned base that one step covers (the
    aligned scan: every lane loads its U vectors once, lanes past the row masked, position 0
    taken from the first lane's own first vector): rows that fill the B x 256 x U vectors
    exactly and rows 1, 64 and 255 vectors short of that, with a NaN at position 0, a NaN in
    the row's last vector, and the extreme value tied at the first and the last position.
    Under a four-workgroup capacity the workgroup-per-row kernel loops over rows."""
    rng = np.random.default_rng(1400 + DTYPES.index(dtype) + 10 * path)
    v = VW[dtype]
    nan = W.to_storage(np.array([np.nan]), dtype)[0]
    B.argreduce_debug_force_path(path)
    for cap in (0, 1024):
        B.argreduce_debug_set_capacity(cap)
        for full in (256, 512, 1024, 2048):
            for short in (0, 1, 64, 255):
                cols = (full - short) * v
                rows = 9
                p = B.argreduce_plan(rows, cols, dtype)
                covered = p["blocks_per_row"] * 256 * p["unroll"]
                if p["path"] != path or covered < full - short:
                    continue
                arr = W.random_rows(rng, rows, cols, dtype, "ties")
                arr[1, 0] = nan
                arr[2, -1] = nan
                arr[3, max(cols - v - 1, 0)] = nan
                arr[4, :] = arr[4, 0]
                arr[5, 0] = arr[5, -1] = W.to_storage(np.array([np.inf]), dtype)[0]
                arr[6, 0] = arr[6, -1] = W.to_storage(np.array([-np.inf]), dtype)[0]
                for op in OPS:
                    check(oracle_lib, arr, dtype, op,
                          f"aligned one step cap={cap} vectors={full - short} plan={p}")


SPAN_WIDTHS = {"f32": [32001, 50257, 202047, 65533, 65534, 65535], "f16": [202047, 50257, 32001],
               "bf16": [151937, 100003], "f64": [100003, 25001]}


def check_banded_rows(oracle_lib, rng, dtype, rows, cols, label, offsets=None):
    """Row r holds values in a band of its own (1000 (r mod 64) plus noise), so an element
    leaking in from the next row would beat the whole row under the max ops and one from the
    previous row under the min ops (except across a wrap of the band, every 64th row); the
    elements before and after the tensor hold +inf for the max ops and -inf for the min ops.
    Every element offset within 16 bytes unless given."""
    import torch

    v = VW[dtype]
    band = 1000.0 * (np.arange(rows)[:, None] % 64) + np.rint(rng.uniform(0, 400, (rows, cols)))
    arr = W.to_storage(band, dtype)
    flat = arr.reshape(-1)
    for offset in (range(v) if offsets is None else offsets):
        for op in OPS:
            poison = W.to_storage(np.array([np.inf if op.startswith("max") else -np.inf]), dtype)
            host = np.concatenate([np.repeat(poison, v + offset), flat, np.repeat(poison, v)])
            buf = to_device(host, dtype)
            t = buf[v + offset: v + offset + flat.size].view(rows, cols)
            assert (t.data_ptr() % 16) == (offset * (16 // v)) % 16
            announce(f"{label} rows={rows} cols={cols} {dtype} offset={offset} op={op}")
            rc, got = run(t, dtype, op)
            assert rc == 0
            want = oracle_lib.argreduce_lastaxis(arr, dtype, op)
            assert np.array_equal(got, want), (rows, cols, dtype, offset, op, got, want)
            del buf, t
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_rows_not_whole_vectors(oracle_lib, dtype):
    """Split rows that start off a 16-byte boundary or end in a partial vector: when one
    step covers every row's vectors, the split kernel reads whole aligned vectors and the
    lanes holding a row's first and last vector mask the elements outside the row (else the
    general scan). Banded rows with poison around the tensor (check_banded_rows); every
    element offset within 16 bytes; one and three rows; widths at, and one or two elements
    past, a whole step ([1,65533..65535] fp32 at U = 1, B = 64)."""
    rng = np.random.default_rng(1600 + DTYPES.index(dtype))
    for cols in SPAN_WIDTHS[dtype]:
        for rows in (1, 3):
            p = B.argreduce_plan(rows, cols, dtype)
            assert p["path"] == B.PATH_SPLIT and p["blocks_per_row"] > 1, p
            check_banded_rows(oracle_lib, rng, dtype, rows, cols, f"split span plan={p}")


# (cols, lanes per row, loads per lane) of lane-group and workgroup-per-row plans for rows that
# are not whole vectors: spans that fill the group or step exactly (f32 61: 16 vectors from a
# 12-byte offset in a group of 16; f16 121 likewise; f32 250: 64 vectors for a wavefront;
# f32 2049: 513 of 1024), spans one vector past it (the general scan: f32 7, f16 63, f16 3,
# f16 8191, and f32 31 and 1023, f16 127, f64 15), 8 loads per lane (the general scan: f64
# 4001), and ordinary fits; and rows of
# whole vectors for a wavefront each (fp32 1024, as [65536,1024]): the aligned scan at
# offset 0, the span or general scan at the others.
SPAN_PATH_WIDTHS = {
    "f32": [(5, 2, 1), (7, 2, 1), (61, 16, 1), (101, 32, 1), (250, 64, 1), (999, 64, 4),
            (1500, 256, 2), (2049, 256, 4), (200, 64, 1), (1024, 64, 4), (1023, 64, 4), (31, 8, 1)],
    "f16": [(3, 1, 1), (63, 8, 1), (65, 16, 1), (121, 16, 1), (1001, 64, 2), (3001, 256, 2),
            (8191, 256, 4), (512, 64, 1), (2048, 64, 4), (127, 16, 1)],
    "bf16": [(65, 16, 1), (250, 32, 1), (3001, 256, 2), (4099, 256, 4), (1024, 64, 2)],
    "f64": [(25, 16, 1), (63, 32, 1), (1001, 256, 2), (4001, 256, 8), (256, 64, 2), (512, 64, 4), (15, 8, 1)],
}


@pytest.mark.parametrize("dtype", DTYPES)
def test_group_and_block_rows_not_whole_vectors(oracle_lib, dtype):
    """Lane-group and workgroup-per-row plans on rows that start off a 16-byte boundary or
    end in a partial vector: the span scan (aligned vector loads, the elements outside the
    row masked) when one step of the group or workgroup covers every row's vectors, else the
    general scan; rows of 16-byte aligned whole vectors take the aligned scan. Banded rows with poison around the tensor, every element offset, one and
    three rows; then a lane-group width with enough rows that the groups loop over rows."""
    rng = np.random.default_rng(1700 + DTYPES.index(dtype))
    for cols, lanes, unroll in SPAN_PATH_WIDTHS[dtype]:
        for rows in (1, 3):
            p = B.argreduce_plan(rows, cols, dtype)
            assert (p["lanes_per_row"], p["blocks_per_row"], p["unroll"]) == (lanes, 1, unroll), p
            check_banded_rows(oracle_lib, rng, dtype, rows, cols, f"group/block span plan={p}")
    cols = {"f32": 61, "f16": 65, "bf16": 65, "f64": 25}[dtype]
    rows = 70001
    p = B.argreduce_plan(rows, cols, dtype)
    assert p["grid_rows"] < rows, p  # the groups loop over rows
    check_banded_rows(oracle_lib, rng, dtype, rows, cols, f"looping span plan={p}", offsets=(0, 1))


@pytest.mark.parametrize("cap", [0, 1024, H200_THREADS])
def test_special_value_fuzz(oracle_lib, hooks, cap):
    """Random rows over {NaN, +-inf, +-max, +-1, +-0, +-subnormal}, and raw bit patterns with
    signalling NaNs planted, under several capacities."""
    rng = np.random.default_rng(1000 + cap % 1013)
    B.argreduce_debug_set_capacity(cap)
    for trial in range(40):
        dtype = DTYPES[trial % 4]
        rows = int(rng.integers(1, 200))
        cols = int(rng.choice([1, 2, 5, 31, 64, 100, 257, 1000, 5000, 33333]))
        kind = ("special", "mixed", "bits")[trial % 3]
        arr = W.random_rows(rng, rows, cols, dtype, kind)
        for op in OPS:
            check(oracle_lib, arr, dtype, op, f"fuzz trial={trial} cap={cap} kind={kind}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_plan_boundaries(oracle_lib, hooks, dtype):
    """Rows at the edges of the split plan's one-step rule: for U = 1, 2, 4, 8 loads per lane,
    the widest row that B <= min(256, device wave / rows) workgroups cover in one step, and
    one element more (the next U, or several steps), for 1, 8 and 32 rows: on this device
    [8, 2^20] and [32, 2^18] fp64 are full device waves of the U = 8 kernel."""
    rng = np.random.default_rng(66 + DTYPES.index(dtype))
    cap_blocks = B.argreduce_plan(1, 1, dtype)["device_threads"] // 256
    for rows in (1, 8, 32):
        bmax = min(256, cap_blocks // rows)
        for u in (1, 2, 4, 8):
            edge = bmax * 256 * u * VW[dtype]
            for cols in (edge, edge + 1):
                p = B.argreduce_plan(rows, cols, dtype)
                # quarter steps in [-25, 25): many ties, exact in every format
                arr = W.to_storage(rng.integers(-100, 100, (rows, cols)) / 4.0, dtype)
                for op in ("max", "min_last"):
                    check(oracle_lib, arr, dtype, op,
                          f"split edge rows={rows} u={u} cols={cols} B={p['blocks_per_row']} "
                          f"U={p['unroll']}")
                if cols == edge:
                    assert p["path"] == B.PATH_SPLIT and p["blocks_per_row"] * 256 * p["unroll"] * VW[dtype] >= cols


@pytest.mark.parametrize("dtype", DTYPES)
def test_widths_straddling_widest_scan_step(oracle_lib, hooks, dtype):
    """cols = S-1, S, S+1 where S is the elements one scan step of a row covers."""
    rng = np.random.default_rng(55)
    for cap in (1024, 0):
        B.argreduce_debug_set_capacity(cap)
        p = B.argreduce_plan(1, 1 << 22, dtype)
        step = p["lanes_per_row"] * p["unroll"] * VW[dtype]
        for cols in (step - 1, step, step + 1, 2 * step + 1):
            if cols > (1 << 24):
                continue
            arr = W.random_rows(rng, 1, cols, dtype, "ties")
            for op in OPS:
                check(oracle_lib, arr, dtype, op, f"straddle cap={cap} step={step} cols={cols}")


def test_scratch_offsets_dirty_and_reuse(oracle_lib):
    import torch

    rng = np.random.default_rng(77)
    w = W.c2_row202048_f32()
    t = to_device(w.data, "f32")
    want = {op: oracle_lib.argreduce_lastaxis(w.data, "f32", op) for op in OPS}
    need = B.argreduce_scratch_bytes(1, 202048, "f32")
    big = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    for off in range(16):
        for op in OPS:
            big.copy_(torch.from_numpy(rng.integers(0, 256, need + 64, dtype=np.uint8)))
            announce(f"scratch offset={off} dirty op={op}")
            rc, got = run(t, "f32", op, scratch=big, scratch_offset=off)
            assert rc == 0 and np.array_equal(got, want[op]), (off, op)
    # the same scratch serves shapes of other sizes in turn
    for rows, cols, dtype in [(32, 202048, "f16"), (1, 32000, "f32"), (8, 202048, "f64")]:
        arr = W.random_rows(rng, rows, cols, dtype, "ties")
        need = B.argreduce_scratch_bytes(rows, cols, dtype)
        if need > big.numel():
            big = torch.empty(need, dtype=torch.uint8, device="cuda")
        for op in OPS:
            check(oracle_lib, arr, dtype, op, "scratch reuse", scratch=big)


def test_undersized_scratch_leaves_output_untouched():
    import torch

    t = to_device(W.c2_row202048_f32().data, "f32")
    need = B.argreduce_scratch_bytes(1, 202048, "f32")
    small = torch.zeros(need - 1, dtype=torch.uint8, device="cuda")
    announce("undersized scratch")
    rc, got = run(t, "f32", "max", scratch=small)
    assert rc == -4
    assert got.tolist() == [-7]


def test_graph_capture_and_replay(oracle_lib):
    """Capture one call per path into a HIP graph; replay with new inputs, with an eager call
    on the same scratch between replays; every replay and every eager call must match the
    oracle (the split path's finalizer clears its published words itself, so a replay, whose
    nonce is the captured one, starts from clean words)."""
    import torch

    rng = np.random.default_rng(31)
    for rows, cols, dtype in [(1, 202048, "f32"), (32, 20000, "bf16"), (300, 4096, "f32"),
                              (4096, 64, "f16")]:
        x = torch.empty((rows, cols), dtype={"f32": torch.float32, "f16": torch.float16,
                                            "bf16": torch.bfloat16}[dtype], device="cuda")
        out = torch.empty(rows, dtype=torch.int64, device="cuda")
        need = B.argreduce_scratch_bytes(rows, cols, dtype)
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        sptr, sbytes = (scratch.data_ptr(), need) if need else (0, 0)
        announce(f"graph warm-up rows={rows} cols={cols} dtype={dtype} need={need}")
        assert B.argreduce_lastaxis(x.data_ptr(), dtype, rows, cols, "max", out.data_ptr(),
                                    sptr, sbytes, torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        announce(f"graph capture rows={rows} cols={cols} dtype={dtype}")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                rc = B.argreduce_lastaxis(x.data_ptr(), dtype, rows, cols, "max", out.data_ptr(),
                                          sptr, sbytes, s.cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        for rep in range(10):
            arr = W.random_rows(rng, rows, cols, dtype, "ties" if rep % 2 else "mixed")
            x.copy_(to_device(arr, dtype))
            torch.cuda.synchronize()
            announce(f"graph replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            want = oracle_lib.argreduce_lastaxis(arr, dtype, "max")
            assert np.array_equal(out.cpu().numpy(), want), (rows, cols, dtype, rep)
            # eager work between replays, on the same scratch
            rc, got = run(x, dtype, "min_last", scratch=scratch if need else None)
            assert rc == 0
            assert np.array_equal(got, oracle_lib.argreduce_lastaxis(arr, dtype, "min_last")), rep
        del g


def test_axis_graph_capture_and_replay(oracle_lib):
    """The middle-axis reduction captured into a HIP graph, split (two dispatches; with
    16-byte and with element loads) and not, replayed on new inputs with eager calls in
    between; every result matches the oracle."""
    import torch

    rng = np.random.default_rng(32)
    for outer, length, inner, dtype in [(1, 1 << 16, 32, "f32"), (1, 1 << 16, 33, "f32"),
                                        (256, 16, 256, "f16")]:
        tdt = {"f32": torch.float32, "f16": torch.float16}[dtype]
        x = torch.empty((outer, length * inner), dtype=tdt, device="cuda")
        out = torch.empty(outer * inner, dtype=torch.int64, device="cuda")
        need = B.argreduce_axis_scratch_bytes(outer, length, inner, dtype)
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        plan = B.argreduce_axis_plan(outer, length, inner, dtype)
        announce(f"axis graph capture shape=({outer},{length},{inner}) {dtype} plan={plan}")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                rc = B.argreduce_axis(x.data_ptr(), dtype, outer, length, inner, "max",
                                      out.data_ptr(), scratch.data_ptr(), need, s.cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        for rep in range(6):
            arr = W.random_rows(rng, outer * length, inner, dtype, "ties").reshape(outer, length, inner)
            x.copy_(to_device(arr.reshape(outer, length * inner), dtype))
            torch.cuda.synchronize()
            announce(f"axis graph replay {rep}")
            g.replay()
            torch.cuda.synchronize()
            want = oracle_lib.argreduce_axis(arr, dtype, "max").reshape(-1)
            assert np.array_equal(out.cpu().numpy(), want), (outer, length, inner, dtype, rep)
            check_axis(oracle_lib, arr, dtype, "min", f"axis eager between replays {rep}")
        del g


def test_torch_wrapper_shapes(oracle_lib):
    import torch
    import argmin_reduction_wide_amd as ar

    rng = np.random.default_rng(5)
    arr = W.random_rows(rng, 6, 5000, "f32", "mixed")
    t = to_device(arr, "f32").view(2, 3, 5000)
    announce("torch wrapper 3-D")
    got = ar.argmax(t)
    assert got.shape == (2, 3) and got.dtype == torch.int64
    assert np.array_equal(got.reshape(-1).cpu().numpy(), oracle_lib.argreduce_lastaxis(arr, "f32", "max"))
    got = ar.argmin(t)
    assert np.array_equal(got.reshape(-1).cpu().numpy(), oracle_lib.argreduce_lastaxis(arr, "f32", "min"))
    with pytest.raises(ValueError):
        ar.argmax(torch.zeros(4, 4))  # CPU tensors are refused, never computed on the host
    # a caller's output must be an int64 CUDA tensor of one element per result, and
    # scratch a CUDA tensor: anything else is refused before a kernel runs
    good = torch.empty(6, dtype=torch.int64, device="cuda")
    assert ar.argmax(t, out=good.view(2, 3)) is not None
    assert np.array_equal(good.cpu().numpy(), oracle_lib.argreduce_lastaxis(arr, "f32", "max"))
    for bad in (torch.empty(5, dtype=torch.int64, device="cuda"),
                torch.empty(6, dtype=torch.int32, device="cuda"),
                torch.empty(12, dtype=torch.int64, device="cuda")[::2],
                torch.empty(6, dtype=torch.int64)):
        sentinel = bad.clone()
        with pytest.raises(ValueError):
            ar.argmax(t, out=bad)
        torch.cuda.synchronize()
        assert torch.equal(bad.cpu(), sentinel.cpu())
    with pytest.raises(ValueError):
        ar.argmin(t, scratch=torch.empty(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        ar.cummax(t, scratch=torch.empty(1 << 16, dtype=torch.uint8))


def test_int32_max_wide_rows():
    """[1, INT32_MAX] and [2, 2^30 + 3] f16 (4 GiB each): zeros with planted +1 / -1 values.
    The expected indices are fixed by the construction (first +1 for ArgMax, first -1 for
    ArgMin); rows * cols exceeds 2^31 in the second shape."""
    import torch

    for rows, cols in [(1, 2 ** 31 - 1), (2, 2 ** 30 + 3)]:
        announce(f"wide rows={rows} cols={cols} f16 alloc")
        x = torch.zeros((rows, cols), dtype=torch.float16, device="cuda")
        want_max, want_min = [], []
        for r in range(rows):
            k1, k2 = cols - 5 - r, cols - 1
            x[r, k1] = 1.0
            x[r, k2] = 1.0
            x[r, cols - 3] = -1.0
            x[r, cols - 2] = -1.0
            want_max.append(k1)
            want_min.append(cols - 3)
        for op, want in (("max", want_max), ("min", want_min)):
            announce(f"wide rows={rows} cols={cols} op={op} plan={B.argreduce_plan(rows, cols, 'f16')}")
            rc, got = run(x, "f16", op)
            assert rc == 0 and got.tolist() == want, (rows, cols, op, got)
        del x
        torch.cuda.empty_cache()


def check_axis(oracle_lib, arr, dtype, op, what, **kw):
    import torch

    announce(f"{what} axis dtype={dtype} op={op} shape={arr.shape} plan="
             f"{B.argreduce_axis_plan(*arr.shape, dtype)}")
    outer, length, inner = arr.shape
    t = to_device(arr.reshape(outer, length * inner), dtype, kw.get("offset", 0))
    need = B.argreduce_axis_scratch_bytes(outer, length, inner, dtype)
    scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    if need and kw.get("dirty"):
        scratch.copy_(torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda"))
    out = torch.full((outer * inner,), -7, dtype=torch.int64, device="cuda")
    rc = B.argreduce_axis(t.data_ptr(), dtype, outer, length, inner, op, out.data_ptr(),
                          scratch.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0, f"{what}: status {rc}"
    got = out.cpu().numpy().reshape(outer, inner)
    want = oracle_lib.argreduce_axis(arr, dtype, op)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{what} {dtype} {op} {arr.shape}: {len(bad)} outputs differ; first "
                           f"{tuple(bad[0])}: got {got[tuple(bad[0])]}, oracle {want[tuple(bad[0])]}")


# inner spans the 4 / 16 / 64-lane tiles of element loads and the 8 / 32 / 64-lane tiles of
# 16-byte loads (an inner row of 16, 32, 48 ... bytes), ragged last tiles, and, with a long
# axis and few outputs, the split over several workgroups with its merge dispatch; (200,
# 256, 63): 200 tiles of element loads, two workgroups each.
AXIS_SHAPES = [(1, 1, 2), (3, 7, 3), (2, 300, 5), (4, 33, 16), (2, 1000, 17), (5, 64, 64),
               (2, 129, 100), (1, 20000, 32), (3, 5000, 4), (1, 70001, 2), (8, 512, 257),
               (2, 700, 256), (1, 3000, 520), (1, 300000, 8), (200, 256, 63)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_axis_shapes_all_ops(oracle_lib, hooks, dtype):
    rng = np.random.default_rng(400 + DTYPES.index(dtype))
    for outer, length, inner in AXIS_SHAPES:
        for kind in ("ties", "mixed", "bits"):
            arr = W.random_rows(rng, outer * length, inner, dtype, kind).reshape(outer, length, inner)
            for op in OPS:
                # offset 1: a base that is not 16-byte aligned takes the element loads
                for offset in (0, 1):
                    check_axis(oracle_lib, arr, dtype, op, f"axis kind={kind} offset={offset}",
                               offset=offset)


@pytest.mark.parametrize("path", [B.PATH_BLOCK, B.PATH_SPLIT])
@pytest.mark.parametrize("cap", [0, 1024, H200_THREADS])
def test_axis_forced_split_and_capacities(oracle_lib, hooks, path, cap):
    rng = np.random.default_rng(500 + path + cap % 89)
    B.argreduce_debug_set_capacity(cap)
    B.argreduce_debug_force_path(path)
    for dtype in DTYPES:
        for outer, length, inner in [(3, 7, 3), (2, 1000, 17), (1, 20000, 32), (6, 300, 70)]:
            arr = W.random_rows(rng, outer * length, inner, dtype, "special").reshape(outer, length, inner)
            for op in OPS:
                check_axis(oracle_lib, arr, dtype, op, f"axis forced={path} cap={cap}", dirty=True)


# Split middle axes (B workgroups per tile, merged by the second dispatch) across its
# shapes: B from 3 to 625 workgroups per tile against 4 to 256 outputs per tile (one to
# eight partials per thread of the merge), every format, ragged last tiles.
SPLIT_AXIS = [(1, 20000, 32, "f32"), (1, 300000, 8, "f32"), (1, 2000000, 4, "f32"),
              (1, 600000, 8, "f64"), (1, 100000, 16, "bf16"), (2, 300000, 24, "f16"),
              (1, 40000, 200, "bf16"), (1, 50000, 264, "f32"), (3, 20000, 136, "f64"),
              (1, 8000, 1000, "f32"), (1, 3000, 520, "f32"), (1, 4096, 4096, "f32"),
              (1, 96, 256, "f32")]


@pytest.mark.parametrize("shape", SPLIT_AXIS, ids=lambda s: "x".join(map(str, s)))
def test_axis_split_shapes(oracle_lib, shape):
    outer, length, inner, dtype = shape
    p = B.argreduce_axis_plan(outer, length, inner, dtype)
    assert p["blocks_per_row"] > 2 and p["dispatches"] == 2, p
    rng = np.random.default_rng(1500 + length % 1000 + inner)
    for kind in ("ties", "special", "bits"):
        arr = W.random_rows(rng, outer * length, inner, dtype, kind).reshape(outer, length, inner)
        for op in OPS:
            check_axis(oracle_lib, arr, dtype, op, f"axis split kind={kind}", dirty=True)


def test_axis_torch_wrapper_dims(oracle_lib):
    import torch
    import argmin_reduction_wide_amd as ar

    rng = np.random.default_rng(9)
    arr = W.random_rows(rng, 4 * 6, 50, "f32", "ties").reshape(4, 6, 50)
    t = to_device(arr.reshape(24, 50), "f32").view(4, 6, 50)
    for dim in (0, 1, 2, -1, -2):
        d = dim % 3
        shp = arr.shape
        outer = int(np.prod(shp[:d])); length = shp[d]; inner = int(np.prod(shp[d + 1:]))
        want = oracle_lib.argreduce_axis(np.ascontiguousarray(arr).reshape(outer, length, inner), "f32", "max")
        announce(f"torch wrapper dim={dim}")
        got = ar.argmax(t, dim=dim)
        assert got.shape == tuple(s for k, s in enumerate(shp) if k != d)
        assert np.array_equal(got.reshape(-1).cpu().numpy(), want.reshape(-1)), dim
        got = ar.argmin(t, dim=dim, select_last_index=True)
        want = oracle_lib.argreduce_axis(np.ascontiguousarray(arr).reshape(outer, length, inner), "f32", "min_last")
        assert np.array_equal(got.reshape(-1).cpu().numpy(), want.reshape(-1)), dim
        kept = ar.argmin(t, dim=dim, select_last_index=True, keepdim=True)
        assert kept.shape == tuple(1 if k == d else s for k, s in enumerate(shp)), (dim, kept.shape)
        assert np.array_equal(kept.reshape(-1).cpu().numpy(), want.reshape(-1)), dim


def test_axis_fuzz(oracle_lib):
    """Random middle-axis shapes (outer, length and inner log-uniform, at most 4M elements),
    formats, input kinds and element offsets of the tensor's start, every op: whatever load
    mode, tile width and split the plan and the launcher choose, the oracle's indices."""
    rng = np.random.default_rng(4242)
    dtypes = ("f32", "f16", "bf16", "f64")
    for trial in range(40):
        dtype = dtypes[trial % 4]
        inner = int(np.exp(rng.uniform(np.log(2), np.log(3000))))
        outer = int(np.exp(rng.uniform(0, np.log(300))))
        most = max(1, (4 << 20) // (inner * outer))
        length = int(np.exp(rng.uniform(0, np.log(min(most, 200000)))))
        kind = ("ties", "special", "bits")[trial % 3]
        offset = (0, 1, 3)[int(rng.integers(0, 3))]
        arr = W.random_rows(rng, outer * length, inner, dtype, kind).reshape(outer, length, inner)
        for op in OPS:
            check_axis(oracle_lib, arr, dtype, op, f"axis fuzz trial={trial} kind={kind} offset={offset}",
                       offset=offset, dirty=True)


def test_axis_element_loads_past_32bit_offsets():
    """[1, 2^21 + 3, 1025] fp16 (4.3 GB): the element offsets from a tile's first output pass
    2^32 bytes, so the kernel takes 64-bit addresses instead of a buffer resource. Zeros with
    values planted so that the expected indices are known by construction: column 1000 has
    its +1 beyond 2^32 bytes and its -1 near the start, column 3 the reverse with its -1 at
    the last position, column 0 a NaN at position 0 (index 0 for every op), column 1024 a NaN
    past 2^32 bytes (never taken); every other column ties throughout."""
    import torch

    length, inner = 2 ** 21 + 3, 1025
    assert length * inner * 2 > 2 ** 32
    p = B.argreduce_axis_plan(1, length, inner, "f16")
    assert p["load_bytes"] == 2, p
    announce(f"axis element loads past 32-bit offsets plan={p}")
    x = torch.zeros((length, inner), dtype=torch.float16, device="cuda")
    x[2097000, 1000] = 1.0
    x[7, 1000] = -1.0
    x[5, 3] = 1.0
    x[length - 1, 3] = -1.0
    x[0, 0] = float("nan")
    x[2 ** 21, 1024] = float("nan")
    planted = {"max": {1000: 2097000, 3: 5}, "max_last": {1000: 2097000, 3: 5},
               "min": {1000: 7, 3: length - 1}, "min_last": {1000: 7, 3: length - 1}}
    out = torch.full((inner,), -7, dtype=torch.int64, device="cuda")
    need = B.argreduce_axis_scratch_bytes(1, length, inner, "f16")
    scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    for op in OPS:
        want = np.full(inner, length - 1 if op.endswith("_last") else 0, dtype=np.int64)
        want[0] = 0
        for col, idx in planted[op].items():
            want[col] = idx
        announce(f"axis past 32-bit offsets op={op}")
        rc = B.argreduce_axis(x.data_ptr(), "f16", 1, length, inner, op, out.data_ptr(),
                              scratch.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert rc == 0
        got = out.cpu().numpy()
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (op, bad[:5], got[bad[:5]], want[bad[:5]])
    del x
    torch.cuda.empty_cache()


def test_axis_workloads_full_size(oracle_lib):
    """The middle-axis bench workloads at full size (16-byte and element loads), every
    output against the oracle."""
    for w in W.config_workloads("axis"):
        outer, length, inner = w.axis_shape
        arr = w.data.reshape(outer, length, inner)
        for op in w.ops + tuple(o + "_last" for o in w.ops):
            check_axis(oracle_lib, arr, w.dtype, op, f"axis workload {w.name}")


def test_bounded_wait_gives_up_cleanly(oracle_lib):
    """The split path's bounded wait, driven from the host with a one-poll limit: every
    output is the oracle's index or -1 (a wait that gave up), every kernel ends, and the
    device's timeout count goes up by exactly the number of rows that came out -1; with the
    default limit restored the same scratch gives exact results again and the count stays."""
    import torch

    rng = np.random.default_rng(77)
    cases = [(1, 202048, "f32"), (32, 202048, "f16"), (3, 500000, "f64"), (40, 65536, "bf16")]
    gave_up = 0
    try:
        B.argreduce_debug_set_spin_limit(1)
        for rows, cols, dtype in cases:
            arr = W.random_rows(rng, rows, cols, dtype, "ties")
            want = oracle_lib.argreduce_lastaxis(arr, dtype, "max")
            t = to_device(arr, dtype)
            need = B.argreduce_scratch_bytes(rows, cols, dtype)
            scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
            for rep in range(5):
                announce(f"one-poll limit rows={rows} cols={cols} dtype={dtype} rep={rep}")
                before = B.argreduce_wait_timeouts()
                rc, got = run(t, dtype, "max", scratch=scratch)
                assert rc == 0
                assert np.all((got == want) | (got == -1)), (rows, cols, dtype, got)
                failed = int(np.count_nonzero(got == -1))
                assert B.argreduce_wait_timeouts() - before == failed, (rows, cols, dtype, failed)
                gave_up += failed
            B.argreduce_debug_set_spin_limit(0)
            before = B.argreduce_wait_timeouts()
            rc, got = run(t, dtype, "max", scratch=scratch)
            assert rc == 0 and np.array_equal(got, want)
            assert B.argreduce_wait_timeouts() == before
            B.argreduce_debug_set_spin_limit(1)
    finally:
        B.argreduce_debug_set_spin_limit(0)
    announce(f"one-poll limit: {gave_up} row waits gave up in all")


def test_streaming_read_hook_covers_every_vector():
    """The read-roofline kernel reads every 16-byte vector exactly where the grid-stride walk
    says: a single word set to the kernel's store pattern is reported by the one workgroup
    whose lanes cover it (unrolled body and ragged tail alike), and by no other."""
    import torch

    pattern = 0x9E3779B9
    for nvec, grid, pos in ((1, 1, 0), (1000, 3, 999), (4096, 4, 1234), (1 << 20, 512, 777777),
                            (1 << 20, 512, (1 << 20) - 1), (5 * 2048 + 17, 2, 5 * 2048 + 3)):
        announce(f"streaming read nvec={nvec} grid={grid} pos={pos}")
        x = torch.zeros(nvec * 4, dtype=torch.int32, device="cuda")
        x[pos * 4 + 2] = pattern - (1 << 32)  # the 32-bit pattern as a signed int32
        sink = torch.zeros(grid, dtype=torch.int32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        assert B.argreduce_debug_launch_read(x.data_ptr(), nvec * 16, sink.data_ptr(), grid, st) == 0
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        block = (pos % (grid * 256)) // 256
        want = np.zeros(grid, dtype=np.uint32)
        want[block] = pattern
        assert np.array_equal(got, want), (nvec, grid, pos, got)


def test_concurrent_streams_and_host_threads(oracle_lib):
    """Split-path calls on two streams at once (separate scratch), then from four host
    threads with a stream each: every result matches the oracle (per-call nonces keep the
    published words of concurrent calls apart)."""
    import threading

    import torch

    rng = np.random.default_rng(88)
    cases = [(4, 202048, "f32"), (2, 300000, "bf16"), (1, 500000, "f16"), (8, 100000, "f32")]
    arrs = [W.random_rows(rng, r, c, d, "ties") for r, c, d in cases]
    wants = [oracle_lib.argreduce_lastaxis(a, d, "max") for a, (_, _, d) in zip(arrs, cases)]
    xs = [to_device(a, d) for a, (_, _, d) in zip(arrs, cases)]
    for (r, c, d) in cases:
        assert B.argreduce_plan(r, c, d)["path"] == B.PATH_SPLIT

    def call(k, stream, reps):
        # the outputs' fills and the scratch are made on the stream the library launches on,
        # so that each fill is ordered before its call (a fill on another stream could land
        # after the call's result) and freed scratch is reused only behind the calls
        r, c, d = cases[k]
        need = B.argreduce_scratch_bytes(r, c, d)
        outs = []
        with torch.cuda.stream(stream):
            scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
            for _ in range(reps):
                out = torch.full((r,), -7, dtype=torch.int64, device="cuda")
                rc = B.argreduce_lastaxis(xs[k].data_ptr(), d, r, c, "max", out.data_ptr(),
                                          scratch.data_ptr(), need, stream.cuda_stream)
                assert rc == 0
                outs.append(out)
        return outs

    announce("two streams, interleaved split calls")
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    o0 = call(0, s0, 20)
    o1 = call(1, s1, 20)
    torch.cuda.synchronize()
    for o in o0:
        assert np.array_equal(o.cpu().numpy(), wants[0])
    for o in o1:
        assert np.array_equal(o.cpu().numpy(), wants[1])

    announce("four host threads, a stream each")
    results, errors = {}, []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            results[k] = call(k, s, 10)
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for k in range(len(cases)):
        for o in results[k]:
            assert np.array_equal(o.cpu().numpy(), wants[k]), k


def test_fast_call_and_ctypes_marshalling_agree(oracle_lib):
    """The same calls through the CPython fast-call module and through ctypes give the
    oracle's results on every path kind (split, workgroup, lane group, middle axis, scan)."""
    import torch

    fast = B.fast()
    assert fast is not None, "the fast-call module is built with the library"
    h = B.lib()
    stream = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(91)
    for rows, cols, dtype, op in [(3, 202048, "f32", "max"), (64, 4096, "f16", "min_last"),
                                  (1000, 64, "bf16", "max"), (2, 300000, "f64", "min")]:
        announce(f"marshalling lastaxis [{rows},{cols}] {dtype} {op}")
        arr = W.random_rows(rng, rows, cols, dtype, "ties")
        x = to_device(arr, dtype)
        need = B.argreduce_scratch_bytes(rows, cols, dtype)
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        want = oracle_lib.argreduce_lastaxis(arr, dtype, op)
        for fn in (fast.argreduce_lastaxis, h.argreduce_lastaxis):
            out = torch.full((rows,), -7, dtype=torch.int64, device="cuda")
            rc = fn(x.data_ptr(), B.DTYPE_NAMES[dtype], rows, cols, B.OP_NAMES[op],
                    out.data_ptr(), scratch.data_ptr(), need, stream)
            torch.cuda.synchronize()
            assert rc == 0 and np.array_equal(out.cpu().numpy(), want), fn

    announce("marshalling axis [4,3000,40] f32 max")
    arr = W.random_rows(rng, 4 * 3000, 40, "f32", "ties").reshape(4, 3000, 40)
    x = to_device(arr, "f32")
    need = B.argreduce_axis_scratch_bytes(4, 3000, 40, "f32")
    scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    want = oracle_lib.argreduce_axis(arr, "f32", "max").reshape(-1)
    for fn in (fast.argreduce_axis, h.argreduce_axis):
        out = torch.full((4 * 40,), -7, dtype=torch.int64, device="cuda")
        rc = fn(x.data_ptr(), B.F32, 4, 3000, 40, B.MAX, out.data_ptr(), scratch.data_ptr(),
                need, stream)
        torch.cuda.synchronize()
        assert rc == 0 and np.array_equal(out.cpu().numpy(), want), fn

    announce("marshalling scan [2,50000] i64 cummax")
    arr = rng.integers(-1000, 1000, size=(2, 50000), dtype=np.int64)
    x = torch.from_numpy(arr.copy()).cuda()
    need = B.argreduce_scan_scratch_bytes(2, 50000, "i64")
    scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    want_v, want_i = oracle_lib.cumulative(arr, "i64", "max")
    for fn in (fast.argreduce_scan_lastaxis, h.argreduce_scan_lastaxis):
        vals = torch.empty_like(x)
        idx = torch.full((2, 50000), -7, dtype=torch.int64, device="cuda")
        rc = fn(x.data_ptr(), B.I64, 2, 50000, B.MAX, vals.data_ptr(), idx.data_ptr(),
                scratch.data_ptr(), need, stream)
        torch.cuda.synchronize()
        assert rc == 0, fn
        assert np.array_equal(idx.cpu().numpy(), want_i.reshape(2, 50000)), fn
        assert np.array_equal(vals.cpu().numpy(), want_v.reshape(2, 50000)), fn


def test_axis_many_partials_planted_columns(oracle_lib, hooks):
    """A long axis with few outputs, split over more than 256 workgroups per tile (the
    merge dispatch's one-output workgroups): planted columns with a leading NaN, all -inf,
    the extremum at the last position, ties at both ends, and NaN everywhere but one
    position, for every op."""
    rng = np.random.default_rng(1201)
    length, inner = 600000, 8
    for dtype in ("f32", "f16", "bf16", "f64"):
        v = W.quantised_normal(rng, (length, inner))
        v[0, 0] = np.nan
        v[:, 1] = -np.inf
        v[-1, 2] = 1e4
        v[0, 3] = v[-1, 3] = 1e4
        v[:, 4] = np.nan
        v[123456, 4] = -3.0
        arr = W.to_storage(v, dtype).reshape(1, length, inner)
        p = B.argreduce_axis_plan(1, length, inner, dtype)
        assert p["blocks_per_row"] > 256, p
        for op in OPS:
            check_axis(oracle_lib, arr, dtype, op, "axis planted columns", dirty=True)
