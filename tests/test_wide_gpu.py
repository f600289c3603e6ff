"""GPU parity of the windowed path for rows wider than INT32_MAX (ARGREDUCE_PATH_WIDE).

The windowed path is forced, with small windows, on rows the CPU oracle handles in
seconds (ragged windows, misaligned rows, NaN and ties at window boundaries, every format
and op); then real rows of 2^31 + k elements run with values planted so that the expected
indices (beyond 2^31) are known by construction. Each case is printed before it runs.
"""
import numpy as np
import pytest

import argmin_reduction_wide_amd.binding as B
from argmin_reduction_wide_amd import workloads as W
from gpu_helpers import announce, check, run, to_device

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16", "f64")
OPS = ("max", "min", "max_last", "min_last")


@pytest.fixture(autouse=True)
def wide_hooks():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU; none is visible"
    yield
    B.argreduce_debug_force_path(B.PATH_AUTO)
    B.argreduce_debug_set_window(0)


@pytest.mark.parametrize("window", [1, 7, 1000, 4096, 65537])
def test_forced_windows_against_oracle(oracle_lib, window):
    rng = np.random.default_rng(1200 + window % 1009)
    B.argreduce_debug_force_path(B.PATH_WIDE)
    assert B.argreduce_debug_set_window(window) == 0
    shapes = [(1, 1), (3, 5), (2, 999), (4, 4097), (1, 20000), (2, 131075)]
    if window == 1:
        shapes = shapes[:4]  # one workgroup per element: keep the grid small
    for dtype in DTYPES:
        for rows, cols in shapes:
            for kind, offset in (("ties", 0), ("special", 1), ("mixed", 3), ("bits", 2)):
                arr = W.random_rows(rng, rows, cols, dtype, kind)
                for op in OPS:
                    check(oracle_lib, arr, dtype, op,
                          f"wide window={window} kind={kind} plan={B.argreduce_plan(rows, cols, dtype)}",
                          offset_elems=offset)


def test_window_boundaries(oracle_lib):
    """NaN as the first element of a later window (an ordinary element there, never taken),
    a leading NaN (position 0 of window 0), and equal extremes in different windows."""
    B.argreduce_debug_force_path(B.PATH_WIDE)
    B.argreduce_debug_set_window(100)
    for dtype in DTYPES:
        nan = W.to_storage(np.array([np.nan]), dtype)[0]
        rows = []
        r = W.to_storage(np.zeros(1000), dtype)
        r[100] = nan
        r[200] = nan
        rows.append(r)  # NaN at window starts
        r = W.to_storage(np.zeros(1000), dtype)
        r[0] = nan
        r[500] = W.to_storage(np.array([5.0]), dtype)[0]
        rows.append(r)  # leading NaN holds
        r = W.to_storage(np.zeros(1000), dtype)
        for k in (150, 450, 999):
            r[k] = W.to_storage(np.array([3.0]), dtype)[0]
        for k in (99, 100, 700):
            r[k] = W.to_storage(np.array([-3.0]), dtype)[0]
        rows.append(r)  # ties across windows
        arr = np.stack(rows)
        for op in OPS:
            got = check(oracle_lib, arr, dtype, op, "wide boundaries")
            want = {"max": [0, 0, 150], "min": [0, 0, 99], "max_last": [999, 0, 999],
                    "min_last": [999, 0, 700]}[op]
            assert got.tolist() == want, (dtype, op, got)


def test_forced_wide_graph_replay(oracle_lib):
    """The windowed path captured into a HIP graph (its partials are rewritten every call)."""
    import torch

    B.argreduce_debug_force_path(B.PATH_WIDE)
    B.argreduce_debug_set_window(5000)
    rng = np.random.default_rng(1300)
    rows, cols, dtype = 3, 60000, "f32"
    x = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    out = torch.empty(rows, dtype=torch.int64, device="cuda")
    need = B.argreduce_scratch_bytes(rows, cols, dtype)
    scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
    announce(f"wide graph capture plan={B.argreduce_plan(rows, cols, dtype)}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rc = B.argreduce_lastaxis(x.data_ptr(), dtype, rows, cols, "min_last", out.data_ptr(),
                                      scratch.data_ptr(), need, s.cuda_stream)
    assert rc == 0
    for rep in range(4):
        arr = W.random_rows(rng, rows, cols, dtype, "ties")
        x.copy_(to_device(arr, dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), oracle_lib.argreduce_lastaxis(arr, dtype, "min_last")), rep


def test_rows_wider_than_int32_max():
    """[1, 2^31 + 1000] and [2, 2^31 + 5] f16 (4 GiB per row): zeros, with +1 planted twice and
    -1 planted twice (one of each below 2^31, one above), a NaN at the first element of the
    second window, and a leading NaN in a separate row. Expected indices by construction."""
    import torch

    for rows, cols in [(1, 2 ** 31 + 1000), (2, 2 ** 31 + 5)]:
        plan = B.argreduce_plan(rows, cols, "f16")
        assert plan["path"] == B.PATH_WIDE
        announce(f"wider than INT32_MAX rows={rows} cols={cols} plan={plan}")
        x = torch.zeros((rows, cols), dtype=torch.float16, device="cuda")
        win = plan["window"]
        want = {op: [] for op in OPS}
        for r in range(rows):
            hi = 2 ** 31 + 2 - r  # beyond INT32_MAX
            lo_max, lo_min = 7 + r, 11 + r
            x[r, lo_max] = 1.0
            x[r, hi] = 1.0
            x[r, lo_min] = -1.0
            x[r, cols - 1] = -1.0
            x[r, win] = float("nan")
            want["max"].append(lo_max)
            want["max_last"].append(hi)
            want["min"].append(lo_min)
            want["min_last"].append(cols - 1)
        for op in OPS:
            rc, got = run(x, "f16", op)
            assert rc == 0 and got.tolist() == want[op], (rows, cols, op, got)
        x[0, 0] = float("nan")  # a leading NaN: index 0 for every op
        for op in OPS:
            rc, got = run(x, "f16", op)
            assert rc == 0 and got[0] == 0, (rows, cols, op, got)
        del x
        torch.cuda.empty_cache()


def test_wide_workload_planted():
    """The bench's 2^31 + 4096 fp16 row: planted ArgMax / ArgMin indices."""
    for w in W.config_workloads("wide"):
        announce(f"wide workload {w.name}: building on the device")
        t = W.device_data(w)
        for op in w.ops:
            announce(f"wide workload {w.name} {op} plan={B.argreduce_plan(w.rows, w.cols, w.dtype)}")
            rc, got = run(t, w.dtype, op)
            assert rc == 0 and got[0] == w.planted[op][0], (w.name, op, got)
        del t
