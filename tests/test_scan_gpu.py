"""GPU parity of cummax / cummin with indices: the HIP library against the CPU oracle, bit for
bit (values as storage bits, int64 indices).

Covers row lengths around the tile size and the look-back window (64 tiles), many rows,
every format (f32, f16, bf16, f64, i32, i64), special values (NaN anywhere, +-inf, +-0,
subnormals, integer extremes), aligned and misaligned buffers, dirty scratch, the page's
workloads at full size, HIP graph capture with replays on new inputs, and the torch
wrapper. Each case is printed before it runs.
"""
import numpy as np
import pytest

import argmin_reduction_wide_amd.binding as B
from argmin_reduction_wide_amd import workloads as W
from gpu_helpers import announce, to_device

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16", "f64", "i32", "i64")
OPS = ("max", "min")
INTS = ("i32", "i64")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU; none is visible"
    B.argreduce_debug_set_capacity(0)
    B.argreduce_debug_force_path(B.PATH_AUTO)


def storage_of(t, dtype: str) -> np.ndarray:
    import torch

    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view({2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def inputs(rng, rows: int, cols: int, dtype: str, kind: str) -> np.ndarray:
    if dtype in INTS:
        return W.random_int_rows(rng, rows, cols, dtype, {"ties": "ties", "special": "full",
                                                          "mixed": "full", "constant": "constant",
                                                          "normal": "full", "bits": "full"}[kind])
    return W.random_rows(rng, rows, cols, dtype, kind)


def run_scan(arr: np.ndarray, dtype: str, op: str, offset: int = 0, dirty: bool = False,
             scratch_offset: int = 0, scratch=None):
    """Call argreduce_scan_lastaxis; returns (status, values storage array, int64 indices)."""
    import torch

    rows, cols = arr.shape
    t = to_device(arr, dtype, offset)
    vals = torch.empty_like(t)
    if offset:  # misaligned outputs too
        vbuf = torch.empty(t.numel() + offset, dtype=t.dtype, device="cuda")
        vals = vbuf[offset:].view(t.shape)
    idx = torch.full((rows, cols), -7, dtype=torch.int64, device="cuda")
    need = B.argreduce_scan_scratch_bytes(rows, cols, dtype)
    assert need != B.SIZE_MAX
    if scratch is None:
        scratch = torch.empty(max(need + scratch_offset, 1), dtype=torch.uint8, device="cuda")
    if dirty and need:
        scratch.copy_(torch.randint(0, 256, scratch.shape, dtype=torch.uint8, device="cuda"))
    rc = B.argreduce_scan_lastaxis(t.data_ptr(), dtype, rows, cols, op, vals.data_ptr(),
                                   idx.data_ptr(), scratch.data_ptr() + scratch_offset, need,
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, storage_of(vals, dtype), idx.cpu().numpy()


def check_scan(oracle_lib, arr: np.ndarray, dtype: str, op: str, what: str, **kw):
    rows, cols = arr.shape
    announce(f"scan {what} dtype={dtype} op={op} shape={arr.shape} {kw} plan="
             f"{B.argreduce_scan_plan(rows, cols, dtype)}")
    rc, got_v, got_i = run_scan(arr, dtype, op, **kw)
    assert rc == 0, f"{what}: status {rc}"
    want_v, want_i = oracle_lib.cumulative(arr, dtype, op)
    bad = np.argwhere(got_i != want_i)
    assert bad.size == 0, (f"{what} {dtype} {op} {arr.shape}: {len(bad)} indices differ; first "
                           f"{tuple(bad[0])}: got {got_i[tuple(bad[0])]}, oracle {want_i[tuple(bad[0])]}")
    badv = np.argwhere(bits(got_v) != bits(want_v))
    assert badv.size == 0, (f"{what} {dtype} {op} {arr.shape}: {len(badv)} values differ; first "
                            f"{tuple(badv[0])}")
    return got_v, got_i


# rows of 1 .. many tiles and across the tile-size choices (a U = 1 tile is 1024 f32 /
# 2048 f16 / 512 64-bit elements, U = 2 twice that, U = 8 eight times), row lengths that are
# not multiples of a 16-byte chunk
SHAPES = [(1, 1), (1, 7), (3, 5), (2, 100), (2, 511), (2, 513), (1, 1023), (1, 1025),
          (4, 2047), (2, 2048), (3, 2049), (1, 4095), (2, 4096), (1, 4097), (2, 8191),
          (1, 8193), (1, 20000), (3, 65536), (1, 65537), (1, 131073), (1, 140001)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_scan_shapes_all_ops(oracle_lib, dtype):
    rng = np.random.default_rng(700 + DTYPES.index(dtype))
    for rows, cols in SHAPES:
        for kind in ("ties", "mixed", "bits"):
            arr = inputs(rng, rows, cols, dtype, kind)
            for op in OPS:
                check_scan(oracle_lib, arr, dtype, op, f"shape kind={kind}")


# (cols one element past a 2-chunk tile, a whole-vector width read at an element offset,
# whole vectors one chunk past a 2-chunk tile)
ONE_TILE_WIDTHS = {"f32": (2049, 4096, 2052), "i32": (2049, 4096, 2052), "f16": (4099, 8192, 4104),
                   "bf16": (4099, 8192, 4104), "f64": (1025, 2048, 1026), "i64": (1025, 2048, 1026)}


@pytest.mark.parametrize("dtype", DTYPES)
def test_scan_many_rows_of_one_element_io_tile(oracle_lib, dtype):
    """Half a device wave of rows (1024) that one tile of 4 chunks per lane holds, where the
    plan takes that one tile (no look-back): rows that are not whole vectors or not 16-byte
    aligned (element loads and stores), and aligned whole-vector rows one chunk past a
    2-chunk tile (16-byte loads and stores); against the oracle, every op."""
    rng = np.random.default_rng(850 + DTYPES.index(dtype))
    odd, whole, vec = ONE_TILE_WIDTHS[dtype]
    for cols, offset in ((odd, 0), (whole, 1), (vec, 0)):
        arr = inputs(rng, 1024, cols, dtype, "ties")
        for op in OPS:
            check_scan(oracle_lib, arr, dtype, op, "one element-I/O tile per row", offset=offset)


def test_scan_fuzz(oracle_lib):
    """Random row counts and lengths (log-uniform, at most 4M elements), every format, input
    kinds, buffers aligned or one element off: whatever tile size, I/O mode and look-back
    the plan chooses, the oracle's values and indices."""
    rng = np.random.default_rng(4343)
    for trial in range(40):
        dtype = DTYPES[trial % len(DTYPES)]
        cols = int(np.exp(rng.uniform(0, np.log(300000))))
        rows = int(np.exp(rng.uniform(0, np.log(max(1, min(3000, (4 << 20) // cols))))))
        kind = ("ties", "mixed", "bits")[trial % 3]
        offset = int(rng.integers(0, 2))
        arr = inputs(rng, rows, cols, dtype, kind)
        for op in OPS:
            check_scan(oracle_lib, arr, dtype, op, f"scan fuzz trial={trial} kind={kind}", offset=offset)


@pytest.mark.parametrize("dtype", DTYPES)
def test_scan_special_values_and_offsets(oracle_lib, dtype):
    """Special-value alphabet (NaN first or anywhere, +-inf, +-0, subnormals; integer
    extremes), constant rows; buffers 16-byte aligned and misaligned by one element; state
    words dirty on entry and at a 16-byte-unaligned scratch offset."""
    rng = np.random.default_rng(800 + DTYPES.index(dtype))
    for rows, cols in [(5, 33), (2, 5000), (1, 70000), (64, 96), (1, 600001)]:
        for kind in ("special", "constant"):
            arr = inputs(rng, rows, cols, dtype, kind)
            if dtype not in INTS and kind == "special":
                arr[0, 0] = W.to_storage(np.array([np.nan]), dtype)[0]  # a leading NaN row
            for op in OPS:
                for offset in (0, 1):
                    check_scan(oracle_lib, arr, dtype, op, f"special kind={kind}", offset=offset,
                               dirty=True, scratch_offset=3)


def test_scan_long_rows_many_windows(oracle_lib):
    """Rows of several hundred tiles: each tile folds the aggregates of the earlier groups of
    64 tiles (published by each group's last tile) and of the earlier tiles of its own
    group, ragged last groups and tiles included."""
    rng = np.random.default_rng(901)
    for dtype, cols in (("f32", 3 << 20), ("i64", 1 << 20), ("f16", 5 << 20), ("f32", 9 << 20)):
        arr = inputs(rng, 1, cols, dtype, "ties")
        for op in OPS:
            check_scan(oracle_lib, arr, dtype, op, "long row")


def test_scan_long_row_tile_sizes(oracle_lib):
    """Rows longer than 64 short tiles take the smallest of U = 2, 4, 8 chunks per lane whose
    grid fits a quarter of a device wave (on MI355X: U = 2 for [1,2^20] fp32 and [1,3*2^19]
    fp16, U = 4 for [1,2^21] fp32 and [1,2^20 - 3] int64, U = 8 for [8,2^18 + 5] fp32 and
    [1,2^21] fp64): rows of several groups of tiles, ragged last tiles, every op."""
    rng = np.random.default_rng(905)
    seen = set()
    for dtype, rows, cols in [("f32", 1, 1 << 20), ("f16", 1, 3 << 19), ("f32", 1, 1 << 21),
                              ("i64", 1, (1 << 20) - 3), ("f32", 8, (1 << 18) + 5),
                              ("f64", 1, 1 << 21)]:
        plan = B.argreduce_scan_plan(rows, cols, dtype)
        seen.add(plan["unroll"])
        arr = inputs(rng, rows, cols, dtype, "ties")
        for op in OPS:
            check_scan(oracle_lib, arr, dtype, op, f"long row U={plan['unroll']} plan={plan}")
    assert {2, 4, 8} <= seen, seen


def test_scan_rows_of_more_than_64_groups(oracle_lib):
    """More than 64 groups of tiles in a row (int64: 4096 elements per tile, so 17100007
    elements are 4175 tiles, 66 groups): the earlier groups' aggregates are folded in two
    rounds of polls, and the row ends in a partial tile of a partial group (an odd length:
    element loads; an even one: 16-byte loads)."""
    rng = np.random.default_rng(903)
    for dtype, cols in (("i64", 17100007), ("f64", 17100006)):
        plan = B.argreduce_scan_plan(1, cols, dtype)
        assert plan["blocks_per_row"] > 65 * 64, plan
        arr = inputs(rng, 1, cols, dtype, "ties")
        for op in OPS:
            check_scan(oracle_lib, arr, dtype, op, f"more than 64 groups, {cols} elements")


def test_scan_workloads_full_size(oracle_lib):
    for w in W.config_workloads("scan"):
        for op in w.ops:
            got_v, got_i = check_scan(oracle_lib, w.data, w.dtype, op, f"workload {w.name}")
            if "starts" in w.planted:  # known by construction: the start of each document
                want = np.zeros(w.cols, dtype=np.int64)
                for s in w.planted["starts"]:
                    want[s:] = s
                assert np.array_equal(got_i[0], want) and np.array_equal(got_v[0], want)


def test_scan_graph_capture_replays(oracle_lib):
    """A captured call (its tile states cleared by a kernel node) replayed on new inputs."""
    import torch

    rng = np.random.default_rng(902)
    for dtype, rows, cols in (("f32", 1, 100000), ("i64", 3, 9000), ("bf16", 2, 30000)):
        announce(f"scan graph dtype={dtype} shape=({rows},{cols})")
        first = inputs(rng, rows, cols, dtype, "ties")
        x = to_device(first, dtype)
        vals = torch.empty_like(x)
        idx = torch.empty((rows, cols), dtype=torch.int64, device="cuda")
        need = B.argreduce_scan_scratch_bytes(rows, cols, dtype)
        scratch = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                rc = B.argreduce_scan_lastaxis(x.data_ptr(), dtype, rows, cols, "max",
                                               vals.data_ptr(), idx.data_ptr(), scratch.data_ptr(),
                                               need, s.cuda_stream)
        assert rc == 0
        for rep in range(4):
            arr = inputs(rng, rows, cols, dtype, "ties" if rep % 2 else "mixed")
            x.copy_(to_device(arr, dtype))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            want_v, want_i = oracle_lib.cumulative(arr, dtype, "max")
            assert np.array_equal(idx.cpu().numpy(), want_i), (dtype, rep)
            assert np.array_equal(bits(storage_of(vals, dtype)), bits(want_v)), (dtype, rep)
            # an eager call in between, on the same scratch
            rc, _, got_i = run_scan(arr, dtype, "min", scratch=scratch)
            assert rc == 0 and np.array_equal(got_i, oracle_lib.cumulative(arr, dtype, "min")[1])


def test_scan_torch_wrapper(oracle_lib):
    import torch

    import argmin_reduction_wide_amd as ar

    rng = np.random.default_rng(903)
    arr = W.random_rows(rng, 6, 5000, "f32", "ties")
    t = to_device(arr, "f32").view(2, 3, 5000)
    announce("scan torch wrapper cummax / cummin on [2,3,5000]")
    v, i = ar.cummax(t)
    want_v, want_i = oracle_lib.cumulative(arr, "f32", "max")
    assert v.shape == t.shape and i.dtype == torch.int64
    assert np.array_equal(i.reshape(6, 5000).cpu().numpy(), want_i)
    assert np.array_equal(v.reshape(6, 5000).cpu().numpy(), want_v)
    v, i = ar.cummin(t, dim=2)
    assert np.array_equal(i.reshape(6, 5000).cpu().numpy(), oracle_lib.cumulative(arr, "f32", "min")[1])
    with pytest.raises(ValueError):
        ar.cummax(t, dim=1)
    ti = torch.arange(65536, device="cuda", dtype=torch.int64)
    v, i = ar.cummax(ti)
    assert torch.equal(v, ti) and torch.equal(i, ti)


def test_scan_bounded_look_back_gives_up_cleanly(oracle_lib):
    """The look-back's bounded wait with a one-poll limit: each index is the oracle's or -1
    (a tile that gave up, or one that needed the aggregate of a group whose last tile gave
    up), every tile with -1 indices is all -1, and
    the device's timeout count goes up by exactly the number of such tiles; with the default
    limit restored the same scratch gives exact results and the count stays."""
    import torch

    rng = np.random.default_rng(904)
    cols = 3 << 20
    arr = inputs(rng, 1, cols, "f32", "ties")
    want_v, want_i = oracle_lib.cumulative(arr, "f32", "max")
    need = B.argreduce_scan_scratch_bytes(1, cols, "f32")
    tile = B.argreduce_scan_plan(1, cols, "f32")["outputs_per_block"]
    scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
    try:
        B.argreduce_debug_set_spin_limit(1)
        for rep in range(3):
            announce(f"scan one-poll limit rep={rep}")
            before = B.argreduce_wait_timeouts()
            rc, _, got_i = run_scan(arr, "f32", "max", scratch=scratch)
            assert rc == 0
            assert np.all((got_i == want_i) | (got_i == -1))
            per_tile = (got_i[0] == -1).reshape(-1, tile)  # cols is a multiple of the tile
            failed = per_tile.any(axis=1)
            assert np.array_equal(per_tile.all(axis=1), failed)
            assert B.argreduce_wait_timeouts() - before == int(failed.sum())
    finally:
        B.argreduce_debug_set_spin_limit(0)
    before = B.argreduce_wait_timeouts()
    rc, got_v, got_i = run_scan(arr, "f32", "max", scratch=scratch)
    assert rc == 0 and np.array_equal(got_i, want_i) and np.array_equal(bits(got_v), bits(want_v))
    assert B.argreduce_wait_timeouts() == before


def test_graph_then_eager_calls_in_a_fresh_process():
    """In a process of its own (so that its nonce counter starts from the beginning): a
    captured multi-tile scan replayed, then the first eager scan on the same scratch, then an
    eager split ArgMax on it, then a replay and an eager scan again; every result bit-exact
    against the oracle. A capture that reused a value of the eager nonce sequence would let
    the eager calls accept the replay's stale state words."""
    import os
    import subprocess
    import sys

    child = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fresh_process_graph_nonce.py")
    announce("fresh process: scan graph replay, then eager calls on the same scratch")
    proc = subprocess.run([sys.executable, "-u", child], capture_output=True, text=True,
                          timeout=300)
    print(proc.stdout, flush=True)
    assert proc.returncode == 0, proc.stdout[-2000:] + proc.stderr[-4000:]
    assert "fresh-process sequence ok" in proc.stdout
