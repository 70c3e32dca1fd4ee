"""bench.py's trace and counter summaries on the CPU, from synthetic rocprofv3
CSVs: only the kernels between a region's two marker launches count, and the
roofline fraction is recomputed from the kernels' medians."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM1 = "void moe::(anonymous namespace)::grouped_gemm_bf16_kernel<0, true, false, false>(args)"
GEMM2 = "void moe::(anonymous namespace)::grouped_gemm_bf16_kernel<1, false, false, false>(args)"
COPY = "void moe::(anonymous namespace)::stream_copy_kernel(args)"
FLOPS = 5.0e12


def bench_line():
    return {"config": {"workload": "w", "tokens": 8, "d": 64, "experts": 2, "top_k": 1, "ffn_width": 64},
            "ms_per_step": 1.0, "steps": 2, "dtype": "bf16",
            "roofline": {"frac": 0.5, "peak": 2500.0, "flops_per_launch": FLOPS}}


def write_trace(path, launches):
    """launches: (name, workgroups, duration ns) in order"""
    t = 1000
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Grid_Size_Y", "Workgroup_Size_Y",
                    "Start_Timestamp", "End_Timestamp"])
        for name, wg, ns in launches:
            w.writerow([name, wg * 256, 256, 1, 1, t, t + ns])
            t += ns + 500


def test_trace_summary_counts_only_the_marked_region(tmp_path):
    # warm-up launches (slow, outside), then region 3 with two calls, then more outside
    launches = [(GEMM1, 100, 9_000_000), (COPY, 3, 1000),
                (GEMM1, 100, 3_000_000), (GEMM2, 50, 1_000_000),
                (GEMM1, 100, 3_200_000), (GEMM2, 50, 1_200_000),
                (COPY, 4, 1000), (GEMM2, 50, 7_000_000)]
    p = tmp_path / "kt.csv"
    write_trace(p, launches)
    text = bench.summarize_trace(str(p), bench_line())
    assert "expert FFN timing loop" in text and "forward steps" not in text
    # medians: GEMM1 3.1 ms, GEMM2 1.1 ms -> 4.2 ms per call
    frac = FLOPS / 4.2e-3 / 1e12 / 2500.0
    assert f"frac {frac:.4f}" in text
    assert "9000.0" not in text and "7000.0" not in text


def test_summary_command_line(tmp_path):
    p = tmp_path / "kt.csv"
    write_trace(p, [(COPY, 1, 1000), (GEMM1, 10, 2_000_000), (GEMM1, 10, 2_000_000), (COPY, 2, 1000)])
    j = tmp_path / "bench.json"
    j.write_text("# a log line\n" + json.dumps(bench_line()) + "\n")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-trace", str(p),
                        "--bench-json", str(j)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "forward steps" in r.stdout and "| 2 |" in r.stdout


def write_pmc(path, counter, launches):
    """launches: (name, workgroups, value)"""
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Grid_Size", "Workgroup_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i, (name, wg, val) in enumerate(launches):
            w.writerow([i + 1, wg * 256, 256, name, counter, val, 0, 1000])


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path):
    gib_kib = (1 << 30) / 1024
    # the counters read half of the copy's bytes (FETCH) and all of them (WRITE)
    seq = lambda rd, wr: [(COPY, 4096, rd * gib_kib), (COPY, 3, 0), (GEMM1, 100, rd * 1e6 / 1024),  # noqa: E731
                          (GEMM2, 50, rd * 2e6 / 1024), (COPY, 4, 0)]
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    write_pmc(f, "FETCH_SIZE", seq(0.5, 1.0))
    write_pmc(w, "WRITE_SIZE", [(n, g, v * 2) for n, g, v in seq(0.5, 1.0)])
    text, rec = bench.summarize_pmc(str(f), str(w), bench_line())
    assert rec["fetch_factor"] == 0.5 and rec["write_factor"] == 1.0
    # reads: (0.5e6 + 1e6) / 0.5 bytes = 3e6; writes (1e6 + 2e6) / 1.0 = 3e6
    assert rec["read_bytes_per_call"] == pytest.approx(3e6, rel=1e-9)
    assert rec["written_bytes_per_call"] == pytest.approx(3e6, rel=1e-9)
    assert "Expert FFN call" in text
