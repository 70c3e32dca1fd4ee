"""Benchmark of one GPU's MoE-layer forward (one JSON line on stdout).

A step is one ``moe_forward`` call on the whole batch: router GEMM, top-k
gating, dispatch queues, grouped SwiGLU expert FFN with the gather fused into
its first GEMM, and the gate-weighted combine.  The default workload is the
Mixtral-shaped layer (T=8192 tokens, d=4096, E=8 experts, top-2, SwiGLU
width 14336, bf16 storage, fp32 accumulation) with seeded synthetic inputs
and random weights; inputs are resident in HBM before timing starts.

Besides the step time it measures, with HIP events on the stream the kernels
run on, the expert-FFN call (the dominant work: 6*k*d*f FLOPs per token),
the dispatch call with the row gather materialised, and the combine, and it
times the CPU oracle on a bounded slice of the same workload.  For bf16
workloads it also times the layer's backward (``moe_backward``: 16*k*d*f
GEMM FLOPs per token) for a seeded output gradient; the transposed weight
layouts it reads are made once beforehand, as after an optimizer step.  With
d and f multiples of 128 it also times the fp8 expert FFN
(``moe_expert_ffn_fp8``: E4M3 codes with per-row power-of-two scales, FP8
MFMA, the quantisation of x and h included) against the dense fp8 peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE layer fwd tokens/s; expert-GEMM TFLOP/s (% MFMA peak); dispatch GB/s"
FFN_SRC = os.path.join(ROOT, "mixture_experts_layer_exclusive_amd", "csrc", "expert_ffn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_ffn_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_8x_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens of the workload the CPU oracle runs for the baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 expert-FFN timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run moe_stream_copy over 1 GiB (the plain copy that calibrates HBM counters)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="no GPU: summarise a rocprofv3 kernel trace (--output-format csv) of a bench.py run, "
                         "per timed region (needs --bench-json)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: HBM-side bytes per expert-FFN call from two rocprofv3 --pmc runs of bench.py "
                         "--copy-calibration (FETCH_SIZE, then WRITE_SIZE); needs --bench-json")
    ap.add_argument("--summarize-mfma", metavar="PMC_CSV",
                    help="no GPU: MFMA utilisation per kernel from a rocprofv3 --pmc MfmaUtil "
                         "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE run of bench.py; needs --bench-json")
    ap.add_argument("--bench-json", help="the JSON line that the traced bench.py run printed")
    ap.add_argument("--traffic-json", help="with --summarize-pmc: also write the traffic record here")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the vendor library's dense bf16 GEMM (torch.mm, hipBLASLt) on the "
                         "shapes of the two expert GEMMs with all T*k rows as one matrix (a measured ceiling)")
    return ap.parse_args()


def src_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per expert-FFN call from the committed counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_src_sha") != src_sha(FFN_SRC):
        return None
    return rec.get("hbm_bytes_per_call")

# Region markers for kernel traces: a tiny moe_stream_copy launch whose
# workgroup count is the marker's number (copies of 16384 * m bytes run on m
# workgroups), issued on the stream outside the timed windows, so that a
# trace summary can pick out exactly the kernels of each timed loop.
REGIONS = {1: "forward steps (the timed moe_forward calls)",
           3: "expert FFN timing loop (the roofline's launches)",
           5: "backward timing loop (moe_backward calls)",
           7: "fp8 expert FFN timing loop (moe_expert_ffn_fp8 calls)"}
MARK_BYTES = 16384
COPY_CAL_WORKGROUPS = 4096  # moe_stream_copy over 1 GiB (--copy-calibration)


class Marker:
    def __init__(self, torch, dev, stream):
        from mixture_experts_layer_exclusive_amd import _lib
        self.lib = _lib.load()
        self.src = torch.zeros(MARK_BYTES * 8, dtype=torch.uint8, device=dev)
        self.dst = torch.empty_like(self.src)
        self.stream = stream

    def __call__(self, m):
        rc = self.lib.moe_stream_copy(self.src.data_ptr(), self.dst.data_ptr(), MARK_BYTES * m,
                                      self.stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"trace marker {m}: status {rc}")


def _short(name):
    import re
    name = name.replace("void ", "").replace("moe::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def _regions(rows, wg_of, name_of):
    """rows in dispatch order -> {first marker: rows strictly between it and the next}"""
    marks = [(i, wg_of(r)) for i, r in enumerate(rows)
             if name_of(r).startswith("stream_copy_kernel") and wg_of(r) <= 8]
    out = {}
    for (i, m), (j, m2) in zip(marks, marks[1:]):
        if m in REGIONS and m2 == m + 1:
            out[m] = rows[i + 1:j]
    return out


def summarize_trace(path, bench):
    import csv
    import statistics as st
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    wg = lambda r: int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])  # noqa: E731
    reg = _regions(rows, wg, lambda r: _short(r["Kernel_Name"]))
    cfg = bench["config"]
    out = [f"Workload: {cfg['workload']} (T={cfg['tokens']}, d={cfg['d']}, E={cfg['experts']}, k={cfg['top_k']}, "
           f"f={cfg['ffn_width']}); the bench line: ms_per_step {bench['ms_per_step']}, roofline.frac "
           f"{bench['roofline']['frac']}.", ""]
    per_call = {}
    for m, name in REGIONS.items():
        if m not in reg:
            continue
        ks = {}
        for r in reg[m]:
            key = (_short(r["Kernel_Name"]), wg(r), int(r["Grid_Size_Y"]) // int(r["Workgroup_Size_Y"]))
            ks.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        calls = {1: bench["steps"]}.get(m, None)
        tot = sum(sum(v) for v in ks.values())
        out += [f"### {name}", "",
                "| kernel | workgroups | launches | min us | median us | mean us | share % |",
                "|---|---|---|---|---|---|---|"]
        for (kn, gx, gy), v in sorted(ks.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"| {kn} | {gx}x{gy} | {len(v)} | {min(v):.1f} | {st.median(v):.1f} | "
                       f"{sum(v) / len(v):.1f} | {100 * sum(v) / tot:.2f} |")
        # launches per call: the least frequent kernel runs once per call
        n_calls = calls or min(len(v) for v in ks.values())
        med = sum(st.median(v) * len(v) / n_calls for v in ks.values())
        mean = tot / n_calls
        per_call[m] = (n_calls, med, mean)
        out += ["", f"{n_calls} calls; kernel time per call: {med:.1f} us from the medians, {mean:.1f} us mean "
                f"(launch gaps not included).", ""]
    pk = bench["roofline"]["peak"]
    if 1 in per_call:
        n_, med, mean = per_call[1]
        out.append(f"Forward step: {mean / 1e3:.4f} ms of kernel time per step against ms_per_step "
                   f"{bench['ms_per_step']} (wall clock, launches included).")
    if 3 in per_call:
        n_, med, mean = per_call[3]
        fl = bench["roofline"]["flops_per_launch"]
        out.append(f"Expert FFN call: {fl / 1e12:.4f} TFLOP (6*T*k*d*f) / {med:.1f} us (sum of the kernels' medians) / "
                   f"{pk:.0f} TFLOP/s = frac {fl / (med * 1e-6) / 1e12 / pk:.4f}; with the mean, "
                   f"{fl / (mean * 1e-6) / 1e12 / pk:.4f}; the bench line (HIP events around the loop): "
                   f"{bench['roofline']['frac']}.")
    if 5 in per_call and bench.get("backward"):
        n_, med, mean = per_call[5]
        fl = bench["backward"]["gemm_flops_per_call"]
        out.append(f"Backward call: {fl / 1e12:.4f} TFLOP (16*T*k*d*f) / {med:.1f} us / {pk:.0f} = frac "
                   f"{fl / (med * 1e-6) / 1e12 / pk:.4f}; the bench line: {bench['backward']['frac_mfma_peak']}.")
    if 7 in per_call and bench.get("fp8_expert_ffn"):
        n_, med, mean = per_call[7]
        fl = bench["fp8_expert_ffn"]["flops_per_call"]
        p8 = bench["fp8_expert_ffn"]["peak"]
        out.append(f"fp8 expert FFN call: {fl / 1e12:.4f} TFLOP / {med:.1f} us / {p8:.0f} = frac "
                   f"{fl / (med * 1e-6) / 1e12 / p8:.4f}; the bench line: {bench['fp8_expert_ffn']['frac_mfma_peak']}.")
    return "\n".join(out) + "\n"


def _pmc_dispatches(path):
    """rocprofv3 --pmc CSV -> one dict per dispatch, in dispatch order: short
    kernel name, workgroups, duration (us) and {counter: value}."""
    import csv
    by = {}
    for r in csv.DictReader(open(path)):
        d = int(r["Dispatch_Id"])
        e = by.setdefault(d, {"name": _short(r["Kernel_Name"]),
                              "wg": int(r["Grid_Size"]) // int(r["Workgroup_Size"]),
                              "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, "c": {}})
        e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [v for _, v in sorted(by.items())]


def summarize_pmc(fetch_csv, write_csv, bench):
    """HBM-side bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB) per
    dispatch, each scaled by what it reads for the 1 GiB moe_stream_copy
    launches of --copy-calibration (read and written bytes known exactly),
    for the expert FFN and backward timing loops."""
    fr, wr = _pmc_dispatches(fetch_csv), _pmc_dispatches(write_csv)
    if [(a["name"], a["wg"]) for a in fr] != [(a["name"], a["wg"]) for a in wr]:
        raise SystemExit("the two counter runs dispatched different kernels")
    cal = [i for i, a in enumerate(fr) if a["name"].startswith("stream_copy_kernel") and a["wg"] == COPY_CAL_WORKGROUPS]
    if not cal:
        raise SystemExit("no 1 GiB moe_stream_copy launches: run bench.py with --copy-calibration")
    gib_kib = (1 << 30) / 1024
    ff = sum(fr[i]["c"]["FETCH_SIZE"] for i in cal) / len(cal) / gib_kib
    wf = sum(wr[i]["c"]["WRITE_SIZE"] for i in cal) / len(cal) / gib_kib
    reg = _regions(list(range(len(fr))), lambda i: fr[i]["wg"], lambda i: fr[i]["name"])
    if 3 not in reg:
        raise SystemExit("no expert FFN timing loop between markers 3 and 4")
    lines = [f"Calibration: {len(cal)} moe_stream_copy launches of exactly 1 GiB; FETCH_SIZE reads {ff:.4f} x the "
             f"bytes they read, WRITE_SIZE {wf:.4f} x the bytes they write. Scaled bytes = counter / factor; "
             "FETCH counts reads that miss the L2 (served by the Infinity Cache or HBM).", ""]
    totals = {}
    for m in (3, 5):
        if m not in reg:
            continue
        agg = {}
        for i in reg[m]:
            e = agg.setdefault((fr[i]["name"], fr[i]["wg"]), [0, 0.0, 0.0])
            e[0] += 1
            e[1] += fr[i]["c"]["FETCH_SIZE"] * 1024 / ff
            e[2] += wr[i]["c"]["WRITE_SIZE"] * 1024 / wf
        n_calls = min(c for c, _, _ in agg.values())
        totals[m] = (n_calls, sum(e[1] for e in agg.values()) / n_calls, sum(e[2] for e in agg.values()) / n_calls)
        lines += [f"### {REGIONS[m]}", "", "| kernel | workgroups | launches | read MB per launch | written MB per launch |",
                  "|---|---|---|---|---|"]
        for (kn, g), (c, rd, wt) in sorted(agg.items(), key=lambda kv: -(kv[1][1] + kv[1][2])):
            lines.append(f"| {kn} | {g} | {c} | {rd / c / 1e6:.1f} | {wt / c / 1e6:.1f} |")
        lines += ["", f"{n_calls} calls: {totals[m][1] / 1e9:.3f} GB read and {totals[m][2] / 1e9:.3f} GB written "
                  "beyond the L2 per call.", ""]
    cfg = bench["config"]
    T, d, E, k, f = cfg["tokens"], cfg["d"], cfg["experts"], cfg["top_k"], cfg["ffn_width"]
    es = 2 if bench["dtype"] == "bf16" else 4
    alg = (3 * E * d * f + T * d + 2 * T * k * f + T * k * d) * es
    n_calls, read, written = totals[3]
    lines.append(f"Expert FFN call: {(read + written) / 1e9:.3f} GB beyond the L2 per call against {alg / 1e9:.3f} GB "
                 f"algorithmic (each expert weight once, x once, h written and read, y_perm written): "
                 f"{(read + written) / alg:.2f} x.")
    rec = {"hbm_bytes_per_call": int(read + written), "read_bytes_per_call": int(read),
           "written_bytes_per_call": int(written), "algorithmic_bytes_per_call": int(alg),
           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4), "workload": cfg["workload"]}
    return "\n".join(lines) + "\n", rec


def summarize_mfma(path):
    """MfmaUtil (rocprofv3's derived counter: SQ_VALU_MFMA_BUSY_CYCLES over
    all SIMDs / (GRBM_GUI_ACTIVE x SIMDs)) per kernel of the forward steps,
    the expert FFN loop, the backward loop and the fp8 expert FFN loop (when
    the run has them), and of the register-only MFMA
    kernel; the clock is GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 / the
    kernel's duration, given for kernels of 500 us or more."""
    ds = _pmc_dispatches(path)
    reg = _regions(ds, lambda a: a["wg"], lambda a: a["name"])
    reg["peak"] = [a for a in ds if a["name"].startswith("mfma_peak_kernel")]
    reg["lib"] = [dict(a, name="vendor library GEMM (" + a["name"][:24] + "...)") for a in ds if "Cijk" in a["name"]]
    lines = []
    for m, title in [(1, REGIONS[1]), (3, REGIONS[3]), (5, REGIONS[5]), (7, REGIONS[7]),
                     ("peak", "register-operand MFMA kernel (moe_mfma_peak)"),
                     ("lib", "the vendor library's dense GEMM on the expert GEMMs' shapes (--library-gemm)")]:
        if not reg.get(m):
            continue
        agg = {}
        for a in reg[m]:
            e = agg.setdefault((a["name"], a["wg"]), [0, 0.0, 0.0, 0.0])
            e[0] += 1
            e[1] += a["us"]
            e[2] += a["c"].get("MfmaUtil", 0.0)
            e[3] += a["c"].get("GRBM_GUI_ACTIVE", 0.0)
        lines += [f"### {title}", "", "| kernel | workgroups | launches | mean us | MfmaUtil % | clock GHz |",
                  "|---|---|---|---|---|---|"]
        for (kn, g), (c, us, mu, ga) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
            clk = f"{ga / 8 / (us * 1e3):.2f}" if us / c >= 500 else "-"
            lines.append(f"| {kn} | {g} | {c} | {us / c:.1f} | {mu / c:.1f} | {clk} |")
        lines.append("")
    return "\n".join(lines)


def summary_mode(args):
    if not args.bench_json:
        raise SystemExit("--bench-json is required")
    bench = json.loads([l for l in open(args.bench_json).read().splitlines() if l.startswith("{")][-1])
    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace, bench))
    if args.summarize_mfma:
        sys.stdout.write(summarize_mfma(args.summarize_mfma))
    if args.summarize_pmc:
        text, rec = summarize_pmc(*args.summarize_pmc, bench)
        sys.stdout.write(text)
        if args.traffic_json:
            rec["kernel_src_sha"] = src_sha(FFN_SRC)
            json.dump(rec, open(args.traffic_json, "w"), indent=1)


def main():
    args = parse()
    if args.summarize_trace or args.summarize_pmc or args.summarize_mfma:
        summary_mode(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(each GPU would run this same layer on its own token shard); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_inputs as mi
    import mixture_experts_layer_exclusive_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = mi.WORKLOADS[args.workload]
    p = spec["problem"]
    tdt = torch.bfloat16 if p.dtype == "bf16" else torch.float32

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    t_gen = time.perf_counter()
    L = mi.make_layer(args.workload, seed=0)
    x, wg, wu, wd = up(L["x"]), up(L["w_gate"]), up(L["w_up"]), up(L["w_down"])
    wr = up(L["w_router"]) if L["w_router"] is not None else None
    lg = up(L["logits"]) if L["logits"] is not None else None
    t_gen = time.perf_counter() - t_gen
    print(f"# inputs generated and uploaded in {t_gen:.1f} s", file=sys.stderr, flush=True)

    prob = moe.problem(p.T, p.d, p.E, p.k, p.f, tdt)
    ws = torch.empty(moe.workspace_size(prob, 3), dtype=torch.uint8, device=dev)
    y = torch.empty(p.T, p.d, dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev)

    mark = Marker(torch, dev, stream)

    def step():
        moe.forward(x, wg, wu, wd, p.k, w_router=wr, logits=lg, ws=ws, y=y)

    for _ in range(args.warmup):
        step()
    mark(1)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mark(2)
    ms_step = wall * 1e3 / args.steps
    ms_step_ev = ev0.elapsed_time(ev1) / args.steps
    tokens_s = p.T / (ms_step / 1e3)
    print(f"# forward: {ms_step:.3f} ms/step wall, {ms_step_ev:.3f} ms/step events",
          file=sys.stderr, flush=True)

    # ---- per-call timings with HIP events on the launch stream ----
    _, inter = moe.forward(x, wg, wu, wd, p.k, w_router=wr, logits=lg, intermediates=True)
    torch.cuda.synchronize()
    ids, gates = inter["topk_ids"], inter["topk_gates"]
    offsets, sa, apos = inter["offsets"], inter["sorted_assign"], inter["assign_pos"]
    n = p.T * p.k
    ffn_ws = torch.empty(moe.workspace_size(prob, 2), dtype=torch.uint8, device=dev)
    disp_ws = torch.empty(max(256, moe.workspace_size(prob, 1)), dtype=torch.uint8, device=dev)
    y_perm = torch.empty(n, p.d, dtype=tdt, device=dev)
    x_perm = torch.empty(n, p.d, dtype=tdt, device=dev)
    disp_out = dict(counts=torch.empty_like(inter["counts"]), offsets=torch.empty_like(offsets),
                    sorted_assign=torch.empty_like(sa), assign_pos=torch.empty_like(apos),
                    x_perm=x_perm)
    y2 = torch.empty_like(y)

    def timed(fn, reps, region=None):
        for _ in range(2):
            fn()
        if region:
            mark(region)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        if region:
            mark(region + 1)
        return a.elapsed_time(b) / reps  # ms

    def timed_cold(fn, reps):
        """Median of single calls, each after reading a 1 GiB buffer (four
        times the 256 MB Infinity Cache), so that the call's inputs come from
        HBM.  The buffer is only read between calls: the lines it leaves in
        the caches are clean, so the call's own writes evict nothing that has
        to be written back first."""
        flush = torch.ones((1 << 30) // 4, dtype=torch.int32, device=dev)
        out = []
        for _ in range(reps + 1):
            flush.max()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        del flush
        return float(sorted(out[1:])[len(out[1:]) // 2])

    reps = max(5, args.steps)
    ms_ffn = timed(lambda: moe.expert_ffn(offsets, wg, wu, wd, p.k, p.T, x=x, sorted_assign=sa,
                                          ws=ffn_ws, y_perm=y_perm), reps, region=3)
    ms_disp = timed(lambda: moe.dispatch(ids, p.E, x=x, with_x_perm=True, ws=disp_ws, out=disp_out), reps)
    ms_comb = timed(lambda: moe.combine(y_perm, apos, gates, y=y2), reps)
    ms_disp_cold = timed_cold(lambda: moe.dispatch(ids, p.E, x=x, with_x_perm=True, ws=disp_ws, out=disp_out),
                              min(reps, 10))
    ms_comb_cold = timed_cold(lambda: moe.combine(y_perm, apos, gates, y=y2), min(reps, 10))
    if lg is None:
        lo = torch.empty(p.T, p.E, dtype=torch.float32, device=dev)
        ms_route = timed(lambda: moe.route(p.k, x=x, w_router=wr, ids=ids, gates=gates, logits_out=lo), reps)
    else:
        ms_route = timed(lambda: moe.route(p.k, logits=lg, ids=ids, gates=gates), reps)

    s = 2 if p.dtype == "bf16" else 4
    ffn_flops = 6.0 * p.T * p.k * p.d * p.f
    ffn_tflops = ffn_flops / (ms_ffn * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_F32_TFLOPS
    disp_bytes = (1 + p.k) * p.T * p.d * s + 12 * n
    comb_bytes = (p.k + 1) * p.T * p.d * s + 8 * n
    disp_gbs = disp_bytes / (ms_disp * 1e-3) / 1e9
    comb_gbs = comb_bytes / (ms_comb * 1e-3) / 1e9
    disp_gbs_cold = disp_bytes / (ms_disp_cold * 1e-3) / 1e9
    comb_gbs_cold = comb_bytes / (ms_comb_cold * 1e-3) / 1e9

    counts = inter["counts"].cpu().numpy()

    # ---- backward of the layer (bf16 only) ----
    bwd = None
    if p.dtype == "bf16" and not args.no_backward:
        dyg = up(mi.make_grad_output(p, seed=0))
        wt = moe.backward_weights(wg, wu, wd)
        bws = torch.empty(moe.workspace_size(prob, 4), dtype=torch.uint8, device=dev)
        gout = moe.backward(x, wg, wu, p.k, inter, dyg, wt, w_router=wr, ws=bws)
        gout = {key: v for key, v in gout.items() if v is not None}
        ms_bwd = timed(lambda: moe.backward(x, wg, wu, p.k, inter, dyg, wt, w_router=wr, ws=bws, out=gout), reps,
                       region=5)
        bwd_flops = 16.0 * p.T * p.k * p.d * p.f
        bwd = {"ms_per_call": round(ms_bwd, 4), "gemm_flops_per_call": bwd_flops,
               "gemm_tflops": round(bwd_flops / (ms_bwd * 1e-3) / 1e12, 2),
               "frac_mfma_peak": round(bwd_flops / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "tokens_per_s": round(p.T / (ms_bwd * 1e-3), 1)}
        print(f"# backward: {ms_bwd:.3f} ms/call", file=sys.stderr, flush=True)
        del dyg, wt, bws, gout

    if args.copy_calibration:
        # six moe_stream_copy launches of exactly 1 GiB each (one untimed):
        # the reference that scales the HBM byte counters
        moe.stream_copy_gbs(dev)

    # ---- measured ceilings: MFMA-only kernel, device copies ----
    mfma_meas = moe.mfma_peak_tflops(dev)
    copy_gbs = moe.stream_copy_gbs(dev)          # this library's copy kernel
    ca = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cb = torch.empty_like(ca)
    ms_copy = timed(lambda: cb.copy_(ca), 5)
    torch_copy_gbs = 2.0 * ca.numel() / (ms_copy * 1e-3) / 1e9
    del ca, cb
    stream_gbs = max(copy_gbs, torch_copy_gbs)

    # ---- the vendor library's dense GEMM on the expert GEMMs' shapes (bf16 only) ----
    lib_gemm = None
    if args.library_gemm and p.dtype == "bf16":
        lib_gemm = {"note": "torch.mm (hipBLASLt), bf16, one dense GEMM with all T*k rows: "
                            "GEMM1 [T*k, d] x [2f, d]^T, GEMM2 [T*k, f] x [d, f]^T; no gather, routing or SwiGLU"}
        for name, (m_, n_, k_) in (("gemm1", (n, 2 * p.f, p.d)), ("gemm2", (n, p.d, p.f))):
            ga = torch.randn(m_, k_, device=dev, dtype=torch.bfloat16)
            gb = torch.randn(n_, k_, device=dev, dtype=torch.bfloat16)
            gc = torch.empty(m_, n_, device=dev, dtype=torch.bfloat16)
            ms_g = timed(lambda: torch.mm(ga, gb.t(), out=gc), reps)
            lib_gemm[name] = {"m_n_k": [m_, n_, k_], "ms": round(ms_g, 4),
                              "tflops": round(2.0 * m_ * n_ * k_ / (ms_g * 1e-3) / 1e12, 1)}
            del ga, gb, gc
        print(f"# library GEMM: {lib_gemm['gemm1']['tflops']} / {lib_gemm['gemm2']['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)

    # ---- fp8 expert FFN (bf16 workloads with d, f multiples of 128) ----
    fp8 = None
    if p.dtype == "bf16" and p.d % 128 == 0 and p.f % 128 == 0 and not args.no_fp8:
        wq = moe.quantize_weights_fp8(wg, wu, wd)
        ws8 = torch.empty(moe.workspace_size(prob, 5), dtype=torch.uint8, device=dev)
        ms_fp8 = timed(lambda: moe.expert_ffn_fp8(offsets, wq, p.k, x, sa, ws=ws8, y_perm=y_perm), reps, region=7)
        fp8_tflops = ffn_flops / (ms_fp8 * 1e-3) / 1e12
        fp8 = {"ms_per_call": round(ms_fp8, 4), "flops_per_call": ffn_flops, "tflops": round(fp8_tflops, 2),
               "peak": PEAK_FP8_TFLOPS, "frac_mfma_peak": round(fp8_tflops / PEAK_FP8_TFLOPS, 4),
               "speedup_vs_bf16": round(ms_ffn / ms_fp8, 3),
               "scheme": "OCP E4M3 codes, power-of-two scale per token (x), per 32 columns of a queue row "
                         "(h, E8M0, applied by the block-scaled MFMA) and per weight row; fp32 accumulation; "
                         "quantisation of x and h included"}
        print(f"# fp8 expert FFN: {ms_fp8:.3f} ms/call", file=sys.stderr, flush=True)
        del wq, ws8

    # ---- the analytic resource model's prediction for this workload ----
    from mixture_experts_layer_exclusive_amd import resource_model as RM
    lay = RM.Layer(p.T, p.d, p.E, p.k, p.f, 2 if p.dtype == "bf16" else 4)
    model = None
    if p.dtype == "bf16":
        pr = RM.predict_times(lay, counts.tolist())
        model = {"expert_ffn_ms": round(pr["expert_ffn"] / 1e3, 4),
                 "expert_ffn_error": round(pr["expert_ffn"] / 1e3 / ms_ffn - 1, 4),
                 "memory_gb": round(RM.memory(lay, backward=True)["total"] / 1e9, 3)}
        if bwd is not None:
            model["backward_ms"] = round(pr["backward"] / 1e3, 4)
            model["backward_error"] = round(pr["backward"] / 1e3 / bwd["ms_per_call"] - 1, 4)

    # ---- CPU oracle baseline on a bounded slice of the same workload ----
    cpu = None
    if not args.no_cpu_baseline:
        del x_perm, y_perm, ffn_ws, disp_ws
        import oracle
        from threadpoolctl import threadpool_info, threadpool_limits
        S = min(args.cpu_tokens, p.T)
        f32 = lambda a: mi.as_f32(a, p.dtype)  # noqa: E731
        xs = f32(L["x"][:S])
        wgs, wus, wds = f32(L["w_gate"]), f32(L["w_up"]), f32(L["w_down"])
        wrs = f32(L["w_router"]) if L["w_router"] is not None else None
        tc = time.perf_counter()
        if L["logits"] is not None:
            oracle.forward(xs, p.k, wgs, wus, wds, logits=L["logits"][:S])
        else:
            oracle.forward(xs, p.k, wgs, wus, wds, w_router=wrs)
        tc = time.perf_counter() - tc
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        del xs
        # the same oracle on one pinned core: routing and queues over all T
        # tokens, the per-token FFN and combine on a seeded token subset,
        # extrapolated linearly (the per-token work does not depend on T)
        S1 = min(64 if p.d * p.f >= (1 << 25) else 256, p.T)
        aff = os.sched_getaffinity(0)
        core = min(aff)
        x_all = f32(L["x"])
        os.sched_setaffinity(0, {core})
        try:
            with threadpool_limits(1):
                t1 = time.perf_counter()
                lg_all = L["logits"] if L["logits"] is not None else oracle.router_logits(x_all, wrs)
                ids_all, _ = oracle.topk_route(lg_all, p.k)
                oracle.dispatch(ids_all, p.E)
                t_route = time.perf_counter() - t1
                tok = mi.sample_tokens(p.T, S1, seed=0)
                t1 = time.perf_counter()
                oracle.forward_tokens(tok, x_all, lg_all, p.k, wgs, wus, wds)
                t_tok = time.perf_counter() - t1
        finally:
            os.sched_setaffinity(0, aff)
        del x_all
        single = {"value": round(p.T / (t_route + t_tok * p.T / S1), 2), "unit": "tokens/s", "cores": 1,
                  "pinned_cpu": core, "route_dispatch_all_tokens_s": round(t_route, 3),
                  "ffn_combine_tokens": S1, "ffn_combine_s": round(t_tok, 3),
                  "extrapolation": "T / (t_route+dispatch(all T) + t_ffn+combine(S tokens) * T / S)"}
        model_name = "unknown"
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model_name = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = {"value": round(S / tc, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"first {S} of {p.T} tokens, whole layer (router GEMM, top-k, queues, "
                         f"SwiGLU FFN, combine) in float64 numpy with {threads} BLAS threads; {tc:.1f} s",
               "host": {"cpu_model": model_name, "logical_cpus": os.cpu_count(),
                        "cpus_in_affinity": len(aff)},
               "single_thread": single}

    traffic = measured_traffic()
    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(d)) expert weights, "
                "N(0,0.02) router; random weights, no checkpoint)",
        "config": {"workload": args.workload, "tokens": p.T, "d": p.d, "experts": p.E,
                   "top_k": p.k, "ffn_width": p.f, "parallelism": "single GPU"},
        "roofline": {"kernel": "expert FFN call (grouped GEMM1 gate/up+SwiGLU, grouped GEMM2 down)",
                     "bound": "mfma", "achieved": round(ffn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(ffn_tflops / peak, 4),
                     "traffic": traffic, "ms_per_launch": round(ms_ffn, 4),
                     "flops_per_launch": ffn_flops},
        "measured_peaks": {
            "mfma_bf16_tflops": round(mfma_meas, 1),
            "note": "moe_mfma_peak: register-operand MFMAs only, at the clock this GPU holds under full matrix "
                    "load; copies of 1 GiB, read + write bytes: moe_stream_copy (this library's copy kernel) "
                    "and torch's copy_; the stream ceiling is the faster of the two",
            "copy_gbs": round(copy_gbs, 1),
            "torch_copy_gbs": round(torch_copy_gbs, 1),
            "stream_ceiling_gbs": round(stream_gbs, 1),
            "expert_gemm_frac_of_measured_mfma": round(ffn_tflops / mfma_meas, 4) if p.dtype == "bf16" else None,
            "dispatch_frac_of_stream_ceiling": round(disp_gbs_cold / stream_gbs, 4),
            "combine_frac_of_stream_ceiling": round(comb_gbs_cold / stream_gbs, 4),
            "library_gemm": lib_gemm},
        "expert_gemm_tflops": round(ffn_tflops, 2),
        "expert_gemm_frac_mfma_peak": round(ffn_tflops / peak, 4),
        "dispatch_gbs": round(disp_gbs_cold, 1),
        "dispatch_frac_hbm_peak": round(disp_gbs_cold / PEAK_HBM_GBS, 4),
        "combine_gbs": round(comb_gbs_cold, 1),
        "combine_frac_hbm_peak": round(comb_gbs_cold / PEAK_HBM_GBS, 4),
        "stage_ms": {"route": round(ms_route, 4), "dispatch_with_x_perm": round(ms_disp_cold, 4),
                     "expert_ffn": round(ms_ffn, 4), "combine": round(ms_comb_cold, 4)},
        "cold_cache_note": "dispatch and combine: median single call after a 1 GiB read, so that x and y_perm "
                           "come from HBM and not from the 256 MB Infinity Cache (dispatch: histogram, scatter "
                           "and gather launches, with the gaps between them)",
        "warm_cache": {"note": "back-to-back calls; x, x_perm and y_perm partly stay in the Infinity Cache",
                       "dispatch_with_x_perm_ms": round(ms_disp, 4), "dispatch_gbs": round(disp_gbs, 1),
                       "combine_ms": round(ms_comb, 4), "combine_gbs": round(comb_gbs, 1)},
        "expert_counts": {"min": int(counts.min()), "max": int(counts.max()),
                          "empty": int((counts == 0).sum())},
        "backward": bwd,
        "fp8_expert_ffn": fp8,
        "resource_model": model,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
