"""Child process of test_scan_gpu.test_graph_then_eager_calls_in_a_fresh_process.

Run as its own process so that the library's per-call nonce counter starts from the
beginning: the first call that takes a nonce is a scan captured into a HIP graph. The graph
is replayed, which leaves the scan's state words (tagged with the captured call's nonce) in
the scratch buffer; then eager calls share that scratch buffer:

  1. capture a scan of rows several tiles long, replay it once;
  2. the first eager scan on the same scratch, on other input;
  3. an eager split ArgMax whose published words overlap the scan's state words;
  4. a second replay on new input, then an eager scan again.

Each result is compared bit for bit with the oracle. Every step is printed before it runs.
Exit status 0 and the line "fresh-process sequence ok" mean every step matched.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def step(msg: str) -> None:
    print(f"[fresh] {msg}", flush=True)


def main() -> int:
    import numpy as np
    import torch

    import argmin_reduction_wide_amd.binding as B
    import oracle
    from argmin_reduction_wide_amd import workloads as W
    from gpu_helpers import to_device

    assert torch.cuda.is_available()
    o = oracle.load()
    rng = np.random.default_rng(905)
    rows, cols, dtype = 2, 100000, "f32"
    plan = B.argreduce_scan_plan(rows, cols, dtype)
    assert plan["blocks_per_row"] > 1, plan
    split_rows, split_cols = 1, 202048
    assert B.argreduce_plan(split_rows, split_cols, dtype)["path"] == B.PATH_SPLIT
    need = max(B.argreduce_scan_scratch_bytes(rows, cols, dtype),
               B.argreduce_scratch_bytes(split_rows, split_cols, dtype))
    scratch = torch.zeros(need, dtype=torch.uint8, device="cuda")
    bits = lambda a: np.ascontiguousarray(a).view(np.uint32)

    def eager_scan(arr, op):
        x = to_device(arr, dtype)
        vals = torch.empty_like(x)
        idx = torch.full((rows, cols), -7, dtype=torch.int64, device="cuda")
        rc = B.argreduce_scan_lastaxis(x.data_ptr(), dtype, rows, cols, op, vals.data_ptr(),
                                       idx.data_ptr(), scratch.data_ptr(), need,
                                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert rc == 0, rc
        want_v, want_i = o.cumulative(arr, dtype, op)
        assert np.array_equal(idx.cpu().numpy(), want_i), f"eager cum{op} indices differ"
        assert np.array_equal(bits(vals.cpu().numpy()), bits(want_v)), f"eager cum{op} values differ"

    step(f"capture a scan [{rows},{cols}] {dtype} ({plan['blocks_per_row']} tiles per row) "
         f"as the process's first nonce-taking call")
    a0 = W.random_rows(rng, rows, cols, dtype, "ties")
    gx = to_device(a0, dtype)
    gvals = torch.empty_like(gx)
    gidx = torch.empty((rows, cols), dtype=torch.int64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rc = B.argreduce_scan_lastaxis(gx.data_ptr(), dtype, rows, cols, "max",
                                           gvals.data_ptr(), gidx.data_ptr(), scratch.data_ptr(),
                                           need, s.cuda_stream)
    assert rc == 0, rc
    torch.cuda.synchronize()

    def replay(arr, what):
        step(f"replay {what}")
        gx.copy_(to_device(arr, dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_v, want_i = o.cumulative(arr, dtype, "max")
        assert np.array_equal(gidx.cpu().numpy(), want_i), f"replay {what}: indices differ"
        assert np.array_equal(bits(gvals.cpu().numpy()), bits(want_v)), f"replay {what}: values differ"

    replay(a0, "1")
    step("first eager scan on the same scratch, other input")
    eager_scan(W.random_rows(rng, rows, cols, dtype, "mixed"), "max")

    replay(W.random_rows(rng, rows, cols, dtype, "ties"), "2")
    step(f"eager split ArgMax [{split_rows},{split_cols}] on the same scratch")
    arr = W.random_rows(rng, split_rows, split_cols, dtype, "ties")
    x = to_device(arr, dtype)
    for op in ("max", "min", "max_last"):
        out = torch.full((split_rows,), -7, dtype=torch.int64, device="cuda")
        rc = B.argreduce_lastaxis(x.data_ptr(), dtype, split_rows, split_cols, op, out.data_ptr(),
                                  scratch.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert rc == 0, rc
        assert np.array_equal(out.cpu().numpy(), o.argreduce_lastaxis(arr, dtype, op)), op

    replay(W.random_rows(rng, rows, cols, dtype, "mixed"), "3")
    step("eager scans (cummax, cummin) on the same scratch after the replay")
    eager_scan(W.random_rows(rng, rows, cols, dtype, "ties"), "max")
    eager_scan(W.random_rows(rng, rows, cols, dtype, "ties"), "min")
    del g
    print("fresh-process sequence ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
