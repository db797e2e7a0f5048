"""Host-only checks of bench.py: the rocprofv3 summaries keep only settled
calls, the GPU count is refused above one, and the timed path of the
benchmark never imports the oracle or the tests package."""
import ast
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_trace_summary_drops_unsettled_calls(tmp_path):
    # Kernel "k": 3 cold calls of 20 us in the first second, then 4 of 10 us.
    rows = []
    t = 0
    for i, d in enumerate([20, 20, 20, 10, 10, 10, 10]):
        start = t if i < 3 else int(1.5e9) + i * 100_000
        rows.append(["\"k\"", start, start + d * 1000])
        t += 200_000
    _write(tmp_path / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           rows)
    s = bench.summarize_trace(str(tmp_path), 1.0)
    assert len(s) == 1 and s[0]["calls"] == 7 and s[0]["steady_calls"] == 4
    assert s[0]["steady_mean_us"] == 10.0
    assert abs(s[0]["mean_us_all"] - 100 / 7) < 1e-9


def test_pmc_summary_sums_per_dispatch(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
           "End_Timestamp"]
    rows = [[1, "k", "FETCH_SIZE", 5, 0, 1000], [1, "k", "FETCH_SIZE", 5, 0, 1000],
            [2, "k", "FETCH_SIZE", 30, int(2e9), int(2e9) + 4000],
            [3, "copy", "FETCH_SIZE", 7, 10, 20]]
    _write(tmp_path / "x_counter_collection.csv", hdr, rows)
    s = {r["kernel"]: r for r in bench.summarize_pmc(str(tmp_path), 1.0)}
    assert s["k"]["dispatches"] == 2 and s["k"]["steady"] == 1
    assert s["k"]["counters"]["FETCH_SIZE"] == 30.0 and s["k"]["mean_us"] == 4.0
    assert s["copy"]["counters"]["FETCH_SIZE"] == 7.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_timed_path_does_not_import_the_oracle():
    # measure() and everything it calls before the CPU-baseline leg import
    # only torch, the library binding and the input generators.
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    fn = {n.name: n for n in tree.body if isinstance(n, ast.FunctionDef)}
    for name in ("measure", "measure_mix", "hold_stream", "roofline_entry", "dispatch_sweep"):
        for node in ast.walk(fn[name]):
            if isinstance(node, (ast.Import, ast.ImportFrom)):
                mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module]
                for m in mods:
                    assert not (m or "").startswith(("oracle", "tests")), (name, m)


def test_dispatch_sweep_shapes():
    # The sweep covers the three families, each shape once, with the leading
    # dimensions the sweep derives from the layouts.
    shapes = bench.sweep_shapes()
    assert len(shapes) == len(set(shapes)) == 134
    fams = {}
    for dtype, la, lb, M, N, K in shapes:
        assert M >= 1 and N >= 1 and K >= 1 and la in ("row", "col") and lb in ("row", "col")
        fams[dtype] = fams.get(dtype, 0) + 1
    assert fams == {"bf16": 100, "f16": 8, "f32": 16, "fp8": 10}
    assert all(lb == "col" for d, la, lb, *_ in shapes if d == "fp8")
