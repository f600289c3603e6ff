"""Host logic of bench.py (CPU only): the algorithmic byte counts the roofline divides, the
source hash that validates committed counter figures, and the summaries that turn
rocprofv3's CSV output into the committed profiles, run on synthetic CSV files written in
rocprofv3's column layout."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

import bench
from argmin_reduction_wide_amd import workloads as W

COUNTER_HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
                  "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
                  "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
                  "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]
STATS_HEADER = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                "StdDev"]
TRACE_HEADER = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id",
                "Kernel_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp"]

COPY = "__amd_rocclr_copyBuffer"
FILL = ("void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned "
        "char>, std::array<char*, 1ul> >(int, at::native::FillFunctor<unsigned char>, "
        "std::array<char*, 1ul>)")


def lib_kernel(name: str) -> str:
    return (f"void argreduce::(anonymous namespace)::{name}<argreduce::F32, 0>(unsigned char "
            f"const*, long*, unsigned int)")


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        wr.writerow(header)
        for r in rows:
            wr.writerow([r.get(h, 0) for h in header])


def fake(name, rows, cols, dtype="f32", kind="argreduce", axis_shape=None, ops=("max",)):
    return SimpleNamespace(name=name, rows=rows, cols=cols, dtype=dtype, kind=kind, ops=ops,
                           axis_shape=axis_shape, nbytes=rows * cols * W.ITEMSIZE[dtype])


# Three workloads of the three byte formulas; the middle-axis one launches a merge dispatch
# after every call, as a split middle-axis plan does.
FAKES = [fake("rows_f32_8x1000", 8, 1000, ops=("max", "min")),
         fake("axis_f32_2x64x16", 2, 64 * 16, axis_shape=(2, 64, 16)),
         fake("scan_f64_1x4096", 1, 4096, dtype="f64", kind="scan")]
KERNEL_OF = {"rows_f32_8x1000": "k_blocks", "axis_f32_2x64x16": "k_axis",
             "scan_f64_1x4096": "k_cum"}


def pmc_run(directory, counter, per_kib, copy_kib, split_first=False):
    """A synthetic --pmc CSV of one counter over the --pmc-pass sequence of FAKES: a torch
    fill, the calibration copy, then PMC_CALLS library calls per (workload, op) with a torch
    fill between workloads. per_kib(w, call) gives a library dispatch's reading."""
    rows, d = [], 0

    def emit(kernel, value, split=False):
        nonlocal d
        d += 1
        parts = [value / 2, value / 2] if split else [value]
        for v in parts:
            rows.append({"Dispatch_Id": d, "Kernel_Name": kernel, "Counter_Name": counter,
                         "Counter_Value": v})

    emit(FILL, 3.0)
    emit(COPY, copy_kib)
    for w in FAKES:
        for op in w.ops:
            for i in range(bench.PMC_CALLS):
                emit(lib_kernel(KERNEL_OF[w.name]), per_kib(w, i), split=split_first and i == 0)
                if w.axis_shape is not None:
                    emit(lib_kernel("k_axis_merge"), 0.25)
        emit(FILL, 1.0)
    write_csv(os.path.join(directory, "host", "run_counter_collection.csv"), COUNTER_HEADER, rows)


def test_algorithmic_bytes_of_the_headline_and_small_config():
    """Input read once plus one int64 per row: [1,202048] fp32 moves 808,192 + 8 bytes and
    [1,32000] fp32 128,000 + 8."""
    assert bench.algorithmic_bytes(W.c2_row202048_f32()) == 808_200
    assert bench.algorithmic_bytes(W.c1_row32000_f32()) == 128_008


def test_algorithmic_bytes_of_middle_axis_and_scan_workloads():
    """A middle-axis reduction writes one index per (outer, inner) pair; a scan reads the
    input, writes a value per element and an int64 index per element."""
    axis = fake("a", 3, 5 * 7, axis_shape=(3, 5, 7))
    assert bench.algorithmic_bytes(axis) == 3 * 35 * 4 + 3 * 7 * 8
    scan = fake("s", 2, 10, dtype="f16", kind="scan")
    assert bench.algorithmic_bytes(scan) == 2 * 20 * 2 + 20 * 8


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow */ }\n"
    b = "int f(int x) { return 2 * x; }"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(b.replace("2", "3"))


def test_source_hash_covers_every_library_source():
    """The hash reads each listed source, and the list holds every kernel, launch and plan
    source of the library."""
    csrc = os.path.join(bench.ROOT, "argmin_reduction_wide_amd", "csrc")
    listed = {os.path.basename(p) for p in bench.KERNEL_SOURCES}
    on_disk = {f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".cpp", ".h"))}
    assert on_disk <= listed, on_disk - listed
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_measured_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("w:max") is None  # no file
    rec = {"source_hash": bench.kernel_source_hash(),
           "kernels": {"w:max": {"traffic_bytes": 1234.6}}}
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("w:max") == 1235
    assert bench.measured_traffic("w:min") is None
    rec["source_hash"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("w:max") is None
    path.write_text("{not json")
    assert bench.measured_traffic("w:max") is None


def test_roofline_fraction():
    r = bench.roofline(808_200, 3.25)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(808_200 / 3.25e-6 / 1e9, abs=0.05)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)


def test_short_kernel_names():
    assert bench._short(lib_kernel("k_split")) == \
        "argreduce::(anonymous namespace)::k_split<argreduce::F32, 0>"
    assert bench._short("argreduce::k_empty()") == "argreduce::k_empty"
    assert bench._short(COPY) == COPY


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch, capsys):
    """The copy kernel reads and writes COPY_BYTES; its readings (half of that in KiB for
    FETCH_SIZE, four fifths for WRITE_SIZE) fix the scale factors, which turn each library
    dispatch's readings into bytes. Merge dispatches and torch kernels between the calls are
    skipped, and a dispatch reported in two rows is summed."""
    monkeypatch.setattr(bench, "pmc_workloads", lambda: [(w, op) for w in FAKES for op in w.ops])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_kib = bench.COPY_BYTES / 1024

    def fetch_kib(w, i):  # the algorithmic input bytes, half-counted like the copy's
        return (bench.algorithmic_bytes(w) - w.rows * 8) / 1024 / 2 + (i % 2) * 0.5

    def write_kib(w, i):
        return 4.0 * 0.8

    pmc_run(str(tmp_path / "fetch"), "FETCH_SIZE", fetch_kib, copy_kib / 2, split_first=True)
    pmc_run(str(tmp_path / "write"), "WRITE_SIZE", write_kib, copy_kib * 0.8)
    assert bench.traffic_summary(str(tmp_path / "fetch"), str(tmp_path / "write")) == 0
    rec = json.loads((tmp_path / "traffic.json").read_text())
    assert rec["source_hash"] == bench.kernel_source_hash()
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.25)
    keys = [f"{w.name}:{op}" for w in FAKES for op in w.ops]
    assert sorted(rec["kernels"]) == sorted(keys)
    for w in FAKES:
        for op in w.ops:
            k = rec["kernels"][f"{w.name}:{op}"]
            assert KERNEL_OF[w.name] in k["kernel"] and "merge" not in k["kernel"]
            assert k["algorithmic_bytes"] == bench.algorithmic_bytes(w)
            read = bench.algorithmic_bytes(w) - w.rows * 8
            assert k["fetch_kib"] == pytest.approx(read / 2048 + 0.25)
            assert k["traffic_bytes"] == pytest.approx(read + 512 + 4096)
    out = capsys.readouterr().out
    assert "fetch factor 2.0000, write factor 1.2500" in out
    assert out.count("| `argreduce::") == len(keys)


def test_traffic_summary_rejects_a_short_pass(tmp_path, monkeypatch):
    """A pass with fewer than PMC_CALLS dispatches of a workload fails instead of shifting
    the assignment of every later workload."""
    monkeypatch.setattr(bench, "pmc_workloads", lambda: [(w, op) for w in FAKES for op in w.ops])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_kib = bench.COPY_BYTES / 1024
    pmc_run(str(tmp_path / "f"), "FETCH_SIZE", lambda w, i: 1.0, copy_kib)
    pmc_run(str(tmp_path / "w"), "WRITE_SIZE", lambda w, i: 1.0, copy_kib)
    monkeypatch.setattr(bench, "PMC_CALLS", bench.PMC_CALLS + 1)
    with pytest.raises(AssertionError):
        bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"))
    assert not (tmp_path / "traffic.json").exists()


def test_counter_summary_averages_per_workload(tmp_path, monkeypatch, capsys):
    monkeypatch.setattr(bench, "pmc_workloads", lambda: [(w, op) for w in FAKES for op in w.ops])
    pmc_run(str(tmp_path / "a"), "SQ_WAVES", lambda w, i: float(i), 1.0)
    pmc_run(str(tmp_path / "b"), "OccupancyPercent", lambda w, i: 40.0 + (i % 2) * 10, 1.0)
    assert bench.counter_summary([str(tmp_path / "a"), str(tmp_path / "b")]) == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| `")]
    assert len(lines) == sum(len(w.ops) for w in FAKES)
    for ln in lines:  # mean of 0..99 and of 40/50 alternating
        assert ln.endswith("| 100 | 49.50 | 45.00 |"), ln


def test_trace_summary_orders_by_total_time_with_medians(tmp_path, capsys):
    d = tmp_path / "trace"
    a, b = lib_kernel("k_split"), "argreduce::k_empty()"
    write_csv(str(d / "h" / "run_kernel_stats.csv"), STATS_HEADER, [
        {"Name": b, "Calls": 3, "TotalDurationNs": 4000, "AverageNs": 1333.3, "Percentage": 20.0,
         "MinNs": 1000, "MaxNs": 2000},
        {"Name": a, "Calls": 4, "TotalDurationNs": 16000, "AverageNs": 4000.0,
         "Percentage": 80.0, "MinNs": 3000, "MaxNs": 6000}])
    trace = []
    for name, durs in ((a, (3000, 6000, 4000, 3000)), (b, (1000, 2000, 1000))):
        for k, dur in enumerate(durs):
            trace.append({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name,
                          "Start_Timestamp": 10_000 * k, "End_Timestamp": 10_000 * k + dur})
    write_csv(str(d / "h" / "run_kernel_trace.csv"), TRACE_HEADER, trace)
    assert bench.trace_summary(str(d)) == 0
    rows = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| `")]
    assert rows[0] == ("| `argreduce::(anonymous namespace)::k_split<argreduce::F32, 0>` | 4 | "
                       "4.000 | 4.000 | 3.000 | 6.000 | 80.00 |")
    assert rows[1] == "| `argreduce::k_empty` | 3 | 1.333 | 1.000 | 1.000 | 2.000 | 20.00 |"


def test_missing_profiler_output_is_an_error(tmp_path):
    with pytest.raises(FileNotFoundError):
        bench.trace_summary(str(tmp_path))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_shape_lines_time_any_shape_and_forced_splits():
    """bench.py --shape: one JSON line per shape with the per-call time, the trials and the
    streaming-read floor; a forced split's geometry shows in its plan, and the automatic
    plan comes back for the next shape."""
    args = [sys.executable, os.path.join(bench.ROOT, "bench.py"), "--steps", "50", "--warmup", "5",
            "--shape", "4,20000,f32", "--shape", "4,20000,f32,min_last,3,2",
            "--shape", "4,20000,f32"]
    r = subprocess.run(args, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [json.loads(x) for x in r.stdout.splitlines() if x.startswith("{")]
    assert len(lines) == 3
    for ln in lines:
        assert ln["shape"] == [4, 20000] and ln["dtype"] == "f32"
        assert ln["us_per_call"] > 0 and ln["read_floor_us"] > 0 and 0 < ln["pct_of_read_floor"]
    assert lines[1]["op"] == "min_last"
    assert (lines[1]["plan"]["blocks_per_row"], lines[1]["plan"]["unroll"]) == (3, 2)
    assert lines[2]["plan"] == lines[0]["plan"]
