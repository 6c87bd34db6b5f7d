"""Benchmark of the block-scaled FP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-rows]
    python bench.py --mode cold --no-headline --no-cpu --rows-only ROW   (profiling runs)
    python bench.py --trace-summary kernel_trace.csv                       (no GPU)

Headline (one JSON line on stdout): the NVFP4 W4A4 GEMM at M=4096, N=4096,
K=7168 -- A and B bf16 ~ N(0,1) from seeds 120/121, quantised on the GPU by
this library's quantiser with the tensor-amax global scales, alpha =
1/(gsA*gsB), bf16 output.  One step = one fp4_gemm launch.  The GPU's clocks
ramp up during the first ~30 ms of sustained load (per-launch time falls from
~270 to ~190 us over the first ~150 launches), so steps run untimed for
CLOCK_RAMP_S seconds first; then W warm-up steps, then K timed steps bracketed
by device synchronisation; value = algorithmic TFLOP/s (2*M*N*K per step).

The same line carries:
  roofline      the GEMM kernel's achieved rate from HIP events on the
                launch stream against the fp16 dense MFMA peak it computes
                with (2.5 PFLOP/s), plus the measured HBM traffic when the
                committed counter summary matches the current kernel source;
  cpu_baseline  the float64 CPU oracle timed on this host on the same inputs;
  rows          the other hot-path rows (quantiser, small-M GEMM, W4A16,
                MXFP4 GEMM, MoE layer, the 4-layer quantise+GEMM pipeline)
                with per-launch times, cold, warm and graph-replayed, and the
                on-box peaks (MFMA loop per dtype, streaming reads cold and
                warm) that every fraction is also reported against;
  gbs_at_m16    the metric's second half: the 16 x 4096 x 7168 GEMM's
                algorithmic bytes over its cold and graph-replayed times.

Cold protocol: before every cold call a 512 MiB fill (twice the 256 MB
memory-side cache) evicts L2 and the MALL; the call is timed alone with HIP
events.  With --mode cold every call of a row's kernels, warm-up included,
follows a fill and no warm or graph timing runs, so that a rocprofv3 kernel
trace of that process holds cold launches only; --trace-summary turns such a
trace into per-kernel median / p10 / p90 durations.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOPS at 4096x4096x7168 (% FP4 MFMA peak); GB/s at M=16"
PEAK = {"f16": 2500.0, "bf16": 2500.0, "fp4": 10100.0, "fp8": 5000.0}  # dense TFLOP/s
HBM_PEAK_GBS = 8000.0
PUBLISHED_TFLOPS = 6549.9  # B300 SM103 CuTe-DSL mm_fp4 at 4096x4096x7168 (context)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-rows", action="store_true", help="only the headline GEMM")
    p.add_argument("--rows-only", default="", help="comma list of rows to run")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain 256 MiB device-to-device copy (3 times), the "
                        "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    p.add_argument("--mode", choices=["full", "cold"], default="full",
                   help="cold: rows time cold calls only (every call after a fill)")
    p.add_argument("--no-headline", action="store_true", help="skip the headline GEMM")
    p.add_argument("--trace-summary", default="",
                   help="summarise a rocprofv3 kernel_trace.csv (per-kernel duration percentiles) and exit")
    p.add_argument("--counter-derived", nargs=2, metavar=("CSVS", "KERNEL"), default=None,
                   help="print derived rates (clock, MFMA pipe busy, ...) of KERNEL from comma-joined "
                        "rocprofv3 SQ counter CSVs of one command, and exit")
    p.add_argument("--counter-summary", default="",
                   help="summarise a rocprofv3 counter_collection.csv (median per dispatch per kernel and "
                        "grid, FETCH_SIZE / WRITE_SIZE scaled by the 256 MiB copy) and exit")
    return p.parse_args()


def counter_summary(path: str) -> str:
    """Markdown table of median counter values per dispatch, per (kernel, grid
    size).  FETCH_SIZE / WRITE_SIZE (KiB) are also scaled to bytes with the
    factor that makes the 256 MiB device copy (__amd_rocclr_copyBuffer, run by
    --copy-calibration) read or write exactly 256 MiB."""
    import csv
    from collections import defaultdict
    vals = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r.get("Grid_Size") or 0), r["Counter_Name"])
            vals[key].append(float(r["Counter_Value"]))
    med = {k: float(np.median(v)) for k, v in vals.items()}
    counts = {k: len(v) for k, v in vals.items()}
    factor = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        # the calibration copy is the largest copyBuffer dispatch (the others are
        # small host-to-device copies of the inputs)
        cands = [v for (name, grid, c), v in med.items() if "copyBuffer" in name and c == ctr and v > 0]
        if cands and max(cands) > 65536:
            factor[ctr] = (256 << 20) / 1024.0 / max(cands)
    lines = ["| kernel | grid | counter | dispatches | median per dispatch | scaled MB |",
             "|---|---|---|---|---|---|"]
    for (name, grid, ctr), v in sorted(med.items(), key=lambda kv: (kv[0][0], kv[0][1], kv[0][2])):
        short = name if len(name) <= 100 else name[:97] + "..."
        mb = f"{v * 1024.0 * factor[ctr] / 1e6:.2f}" if ctr in factor else ""
        lines.append(f"| `{short}` | {grid} | {ctr} | {counts[(name, grid, ctr)]} | {v:.1f} | {mb} |")
    if factor:
        lines.append("")
        lines.append("Copy calibration factors (bytes per counter KiB / 1024): " +
                     ", ".join(f"{k} {v:.4f}" for k, v in sorted(factor.items())))
    return "\n".join(lines)


def counter_derived(paths: str, kernel: str, cus: int = 256) -> str:
    """Per-dispatch rates of one kernel from rocprofv3 SQ counter CSVs (a
    comma-joined list of passes of the same command, matched by dispatch
    order), medians over dispatches:
      * effective clock = SQ_BUSY_CU_CYCLES / CUs / kernel duration (the
        counter sums the busy cycles of every CU);
      * MFMA pipe busy = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x CUs) over the
        per-CU busy cycles;
      * VALU instructions per MFMA; LDS busy = SQ_LDS_IDX_ACTIVE per CU over
        the busy cycles; TA address / command FIFO full likewise; waves'
        waiting share = SQ_WAIT_ANY / SQ_WAVE_CYCLES (both in quad-cycles)."""
    import csv
    per = []
    for path in paths.split(","):
        by = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel not in r["Kernel_Name"]:
                    continue
                d = by.setdefault(int(r["Dispatch_Id"]), {})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
                d["dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.append([by[k] for k in sorted(by)])
    n = min(len(p) for p in per)
    rows = []
    for i in range(n):
        d = {}
        for p in per:
            d.update(p[i])
        rows.append(d)
    out = {"dispatches": n, "median duration us": float(np.median([d["dur_us"] for d in rows]))}

    def add(name, fn):
        try:
            out[name] = float(np.median([fn(d) for d in rows]))
        except KeyError:
            pass
    add("effective clock GHz", lambda d: d["SQ_BUSY_CU_CYCLES"] / cus / (d["dur_us"] * 1e3))
    add("MFMA pipe busy (fraction of CU busy cycles)",
        lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * cus) / (d["SQ_BUSY_CU_CYCLES"] / cus))
    add("VALU instructions per MFMA", lambda d: d["SQ_INSTS_VALU"] / d["SQ_INSTS_MFMA"])
    add("LDS instructions per MFMA", lambda d: d["SQ_INSTS_LDS"] / d["SQ_INSTS_MFMA"])
    busy = float(np.median([d["SQ_BUSY_CU_CYCLES"] / cus for d in rows])) if "SQ_BUSY_CU_CYCLES" in rows[0] else None
    if busy:
        add("LDS busy (fraction)", lambda d: d["SQ_LDS_IDX_ACTIVE"] / cus / busy)
        add("TA address FIFO full (fraction)", lambda d: d["SQ_VMEM_TA_ADDR_FIFO_FULL"] / cus / busy)
        add("TA command FIFO full (fraction)", lambda d: d["SQ_VMEM_TA_CMD_FIFO_FULL"] / cus / busy)
    add("waves' waiting share", lambda d: d["SQ_WAIT_ANY"] / d["SQ_WAVE_CYCLES"])
    lines = ["| quantity | median |", "|---|---|"]
    lines += [f"| {k} | {v:.4g} |" for k, v in out.items()]
    return "\n".join(lines)


def trace_summary(path: str) -> str:
    """Markdown table of kernel durations (us) per (kernel name, grid size) from
    a rocprofv3 --kernel-trace CSV: launches, median, p10, p90, min, max, mean."""
    import csv
    from collections import defaultdict
    dur = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("KernelName") or r.get("Name")
            grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            dur[(name, grid)].append((t1 - t0) / 1e3)
    lines = ["| kernel | grid (threads) | launches | median us | p10 | p90 | min | max | mean |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        a = np.array(v)
        short = name if len(name) <= 110 else name[:107] + "..."
        lines.append(f"| `{short}` | {grid} | {a.size} | {np.median(a):.2f} | {np.percentile(a, 10):.2f} | "
                     f"{np.percentile(a, 90):.2f} | {a.min():.2f} | {a.max():.2f} | {a.mean():.2f} |")
    return "\n".join(lines)


def src_sha(names: str) -> str:
    """First 16 hex digits of the SHA-256 of the named csrc files (a '+'-joined
    list), concatenated in that order."""
    h = hashlib.sha256()
    for name in names.split("+"):
        with open(os.path.join(ROOT, "block_scaled_fp4_e2m1_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the headline kernel's source files: its body and the shared dequantise-once core
TRAFFIC_SOURCES = "gemm_nvfp4.hip+nvfp4_f16core.h"


def stored_traffic(kernel_key: str, source: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    e = tab.get(kernel_key)
    if not e or e.get("source_sha") != src_sha(source):
        return None
    return e.get("bytes_per_launch")


class Timer:
    """Per-launch durations with HIP events recorded on the current stream.

    cold_only: every call (warm-up included) follows a flush, and warm / graph
    timings are skipped (they return None)."""

    def __init__(self, torch, cold_only=False):
        self.torch = torch
        self.cold_only = cold_only
        self.flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")

    def graph(self, fn, calls=20, reps=5):
        """`calls` back-to-back calls captured in one HIP graph and replayed
        `reps` times between two events: the GPU time per call without the
        host's per-launch cost (which exceeds a few-microsecond kernel).  The
        replayed result is checked against the eager result of the same call
        by the caller through `check`."""
        if self.cold_only:
            return None
        t = self.torch
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(side):
            for _ in range(3):
                fn()
        t.cuda.current_stream().wait_stream(side)
        t.cuda.synchronize()
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g):
            for _ in range(calls):
                fn()
        g.replay()
        t.cuda.synchronize()
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
        del g
        return {"median_us": us, "graph_replay": True, "calls_per_graph": calls}

    def run(self, fn, iters=20, warmup=3, cold=False):
        """cold: each call timed alone after a 512 MiB fill that evicts L2 and the
        256 MB MALL (median/p10/p90 of per-call event times; the fill keeps the
        GPU busy while the host enqueues the call).  warm: `iters` calls back to
        back between two events (their mean), as a pipeline would issue them --
        for kernels of a few microseconds this is bounded by the host's launch
        cost; `graph` gives the GPU time."""
        t = self.torch
        if self.cold_only and not cold:
            return None
        for _ in range(warmup):
            if cold and self.cold_only:
                self.flush.zero_()
            fn()
        t.cuda.synchronize()
        if not cold:
            e0 = t.cuda.Event(enable_timing=True)
            e1 = t.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / iters
            return {"median_us": us, "mean_back_to_back": True}
        times = []
        for _ in range(iters):
            self.flush.zero_()
            e0 = t.cuda.Event(enable_timing=True)
            e1 = t.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        a = np.array(times)
        return {"median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
                "p90_us": float(np.percentile(a, 90))}


# untimed steps before the warm-up steps: the clocks reach steady state
CLOCK_RAMP_S = 0.3


def main():
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.counter_derived:
        print(counter_derived(args.counter_derived[0], args.counter_derived[1]))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_scaled_fp4_e2m1_amd as bs
    from block_scaled_fp4_e2m1_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {"metric": METRIC}
    head = None
    if not args.no_headline:
        head = headline(torch, bs, synth, bf16, args)
        out.update(head["json"])

    # ---------------------------------------------------------------- other rows
    if not args.no_rows:
        only = [r for r in args.rows_only.split(",") if r]
        rows = run_rows(torch, bs, synth, Timer(torch, cold_only=args.mode == "cold"), only)
        out["rows"] = rows
        peaks = rows.get("peaks")
        if head is not None and peaks:
            rf = out["roofline"]
            # the fp16 MFMA rate measured with the operand data this path
            # multiplies (E2M1 x E4M3 products that change every MFMA): the
            # power-limited part's realistic ceiling for the exact NVFP4 GEMM
            mp = peaks["mfma_tflops"].get("f16_nvfp4_products_changing", peaks["mfma_tflops"]["f16"])
            rf["measured_peak"] = mp
            rf["measured_peak_kind"] = ("f16_nvfp4_products_changing"
                                        if "f16_nvfp4_products_changing" in peaks["mfma_tflops"] else "f16")
            rf["frac_of_measured_peak"] = round(rf["achieved"] / mp, 4)
        mx = rows.get("mxfp4_gemm_4096x4096x7168")
        if mx and peaks and "fp4_random_changing" in peaks["mfma_tflops"]:
            # against the FP4 MFMA rate with operands that change every MFMA
            for k in ("warm", "cold"):
                if mx.get(k):
                    mx[k]["frac_of_measured_fp4_changing"] = round(
                        mx[k]["tflops"] / peaks["mfma_tflops"]["fp4_random_changing"], 4)
        m16 = rows.get("nvfp4_gemm_16x4096x7168")
        if m16 and head is not None:
            g = {"cold_gbs": m16["cold"]["gbs"], "cold_frac_hbm": m16["cold"]["frac_hbm"],
                 "cold_us": round(m16["cold"]["median_us"], 3)}
            if m16.get("graph"):
                g.update({"graph_gbs": m16["graph"]["gbs"], "graph_frac_hbm": m16["graph"]["frac_hbm"],
                          "graph_us": round(m16["graph"]["median_us"], 3),
                          "note": "graph replay keeps the 16.7 MB weights in the 256 MB memory-side cache"})
            if peaks:
                g["cold_read_floor_us"] = peaks["read"]["16.7MB_cold"]["median_us"]
                g["cold_vs_read_floor"] = round(m16["cold"]["median_us"] / peaks["read"]["16.7MB_cold"]["median_us"], 3)
            # the metric's second half sits right after the value so that a truncated line keeps it
            keys = list(out.keys())
            i = keys.index("unit") + 1
            out = {k: out[k] for k in keys[:i]} | {"gbs_at_m16": g} | {k: out[k] for k in keys[i:]}

    # ---------------------------------------------------------------- CPU oracle
    if not args.no_cpu and head is not None:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(torch, bs, synth, bf16, head["inputs"])

    print(json.dumps(out), flush=True)


def headline(torch, bs, synth, bf16, args):
    """The NVFP4 GEMM at 4096 x 4096 x 7168: K launches between two HIP events
    on the launch stream after the clock ramp and W warm-up launches."""
    dev = "cuda:0"
    M, N, K = 4096, 4096, 7168
    a = bf16(synth.bf16_normal(120, (M, K)))
    b = bf16(synth.bf16_normal(121, (N, K)))
    gsa, gsb = bs.global_scale(a), bs.global_scale(b)
    aq, sfa = bs.quantize(a, "nvfp4", gs=gsa)
    bq, sfb = bs.quantize(b, "nvfp4", gs=gsb)
    del a, b
    g = torch.cat([gsa, gsb]).cpu().numpy()
    alpha = torch.tensor([np.float32(1.0) / np.float32(g[0] * g[1])], dtype=torch.float32, device=dev)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step():
        bs.gemm(aq, sfa, bq, sfb, alpha, out=D)

    print(f"[bench] headline: {CLOCK_RAMP_S} s clock ramp, {args.warmup} warm-up + {args.steps} timed steps",
          file=sys.stderr, flush=True)
    t_ramp = time.perf_counter()
    while time.perf_counter() - t_ramp < CLOCK_RAMP_S:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    flops = 2.0 * M * N * K
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    alg_bytes = M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + 4 + 2 * M * N

    traffic = stored_traffic("nvfp4_gemm_4096x4096x7168", TRAFFIC_SOURCES)
    roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK["f16"], "unit": "TFLOP/s",
                "frac": round(tflops / PEAK["f16"], 4), "traffic": traffic,
                "frac_of_fp4_peak": round(tflops / PEAK["fp4"], 4),
                "algorithmic_bytes": alg_bytes}
    js = {
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PUBLISHED_TFLOPS, 4),
        "vs_baseline_ref": "B300 SM103 CuTe-DSL mm_fp4, 6549.9 TFLOPS (other hardware; context)",
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "nvfp4_gemm_4096x4096x7168", "M": M, "N": N, "K": K,
                   "operands": "NVFP4 (E2M1 + E4M3/16 + fp32 alpha)", "output": "bf16",
                   "mfma": "v_mfma_f32_32x32x16_f16 on exactly dequantised operands",
                   "timed_wall_s": round(wall, 4), "untimed_clock_ramp_s": CLOCK_RAMP_S},
        "roofline": roofline,
    }
    return {"json": js, "inputs": (aq, sfa, bq, sfb, alpha, D)}


def _nv_bytes(M, N, K):
    return M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + 4 + 2 * M * N


def _rate(t, flops=None, nbytes=None):
    if t is None:
        return None
    r = dict(t)
    us = t["median_us"]
    if flops:
        r["tflops"] = round(flops / us / 1e6, 2)
        r["frac_f16_peak"] = round(flops / us / 1e6 / PEAK["f16"], 4)
        r["frac_fp4_peak"] = round(flops / us / 1e6 / PEAK["fp4"], 4)
    if nbytes:
        r["gbs"] = round(nbytes / us / 1e3, 1)
        r["frac_hbm"] = round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)
    return r


def run_rows(torch, bs, synth, timer, only):
    dev = "cuda:0"

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def want(name):
        if only and name not in only:
            return False
        print(f"[bench] row {name}", file=sys.stderr, flush=True)
        return True

    rows = {}

    def nv_inputs(M, N, K, sa, sb, b_std=1.0, outliers=False):
        a = bf16(synth.bf16_normal_with_outliers(sa, sa + 1000, (M, K)) if outliers
                 else synth.bf16_normal(sa, (M, K)))
        b = bf16(synth.bf16_normal(sb, (N, K), b_std))
        gsa, gsb = bs.global_scale(a), bs.global_scale(b)
        aq, sfa = bs.quantize(a, "nvfp4", gs=gsa)
        bq, sfb = bs.quantize(b, "nvfp4", gs=gsb)
        g = torch.cat([gsa, gsb]).cpu().numpy()
        alpha = torch.tensor([np.float32(1.0) / np.float32(g[0] * g[1])], device=dev)
        return a, gsa, aq, sfa, bq, sfb, alpha

    # On-box peaks: the MFMA loop per dtype (registers only) and streaming reads
    # of the M=16 workload's byte count and of 256 MiB, cold (after the fill, as
    # every cold row) and warm (back to back: the 16.7 MB read then runs from
    # the memory-side cache).
    if want("peaks"):
        import ctypes
        from block_scaled_fp4_e2m1_amd import binding as B
        lib = bs.load()
        stream = lambda: B._stream(torch.device(dev))   # the current stream (a capture stream in a graph)
        mf = {}
        for kind, name, iters in ((0, "f16", 4096), (1, "bf16", 4096), (2, "fp8", 2048), (3, "fp4", 1024),
                                  (4, "f16_3bit_operands", 4096), (5, "bf16_3bit_operands", 4096),
                                  (6, "fp4_random_changing", 1024), (7, "f16_nvfp4_products_changing", 4096)):
            fn = lambda: B._check(lib.bsfp4_probe_mfma(kind, iters, stream()), "probe_mfma")
            t = timer.run(fn, iters=10, warmup=3)
            if t is not None:
                mf[name] = round(lib.bsfp4_probe_mfma_flops(kind, iters) / t["median_us"] / 1e6, 1)
        rd = {}
        for label, nbytes in (("16.7MB", 16710672), ("256MiB", 256 << 20)):
            buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            buf.fill_(1)
            fn = lambda: B._check(lib.bsfp4_probe_read(B._p(buf), nbytes, stream()), "probe_read")
            c = timer.run(fn, cold=True)
            rd[f"{label}_cold"] = {"median_us": round(c["median_us"], 3), "p10_us": round(c["p10_us"], 3),
                                   "p90_us": round(c["p90_us"], 3),
                                   "gbs": round(nbytes / c["median_us"] / 1e3, 1)}
            w = timer.run(fn, iters=20)
            if w is not None:
                rd[f"{label}_warm"] = {"median_us": round(w["median_us"], 3),
                                       "gbs": round(nbytes / w["median_us"] / 1e3, 1)}
            gr = timer.graph(fn)
            if gr is not None:
                rd[f"{label}_graph"] = {"median_us": round(gr["median_us"], 3),
                                        "gbs": round(nbytes / gr["median_us"] / 1e3, 1)}
            del buf
        rows["peaks"] = {"mfma_tflops": mf, "read": rd,
                         "published": {"mfma_tflops": {"f16": PEAK["f16"], "bf16": PEAK["bf16"], "fp8": PEAK["fp8"],
                                                       "fp4": PEAK["fp4"]}, "hbm_gbs": HBM_PEAK_GBS},
                         "note": "MFMA: 8 independent accumulators per wave, register operands (the same "
                                 "operands every MFMA, except the *_changing kinds, which rotate four A and four "
                                 "B registers of random data as a GEMM does); read: 128-bit loads, 4 in flight "
                                 "per lane; cold = after a 512 MiB fill"}

    # a3/a4 at the memory-bound workload: M=16, N=4096, K=7168 (HBM roofline)
    if want("nvfp4_gemm_16x4096x7168"):
        M, N, K = 16, 4096, 7168
        _, _, aq, sfa, bq, sfb, alpha = nv_inputs(M, N, K, 100, 101)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fn = lambda: bs.gemm(aq, sfa, bq, sfb, alpha, out=D)
        fn()
        eager = D.clone()
        rows["nvfp4_gemm_16x4096x7168"] = {
            "cold": _rate(timer.run(fn, cold=True), 2.0 * M * N * K, _nv_bytes(M, N, K)),
            "warm": _rate(timer.run(fn), 2.0 * M * N * K, _nv_bytes(M, N, K)),
            "graph": _rate(timer.graph(fn), 2.0 * M * N * K, _nv_bytes(M, N, K)),
            "graph_matches_eager": bool(torch.equal(D, eager)),
            "bound": "hbm", "algorithmic_bytes": _nv_bytes(M, N, K)}

    # a3 sweep at N=4096, K=7168
    if want("nvfp4_gemm_sweep"):
        sweep = {}
        for i, M in enumerate([1, 64, 512, 2048]):
            N, K = 4096, 7168
            _, _, aq, sfa, bq, sfb, alpha = nv_inputs(M, N, K, 122 + i, 121)
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fn = lambda: bs.gemm(aq, sfa, bq, sfb, alpha, out=D)
            sweep[f"M={M}"] = {"cold": _rate(timer.run(fn, cold=True), 2.0 * M * N * K, _nv_bytes(M, N, K)),
                               "graph": _rate(timer.graph(fn), 2.0 * M * N * K, _nv_bytes(M, N, K))}
        rows["nvfp4_gemm_sweep"] = sweep

    # a1 + a3: quantise bf16 activations, then the NVFP4 GEMM (M=256, N=14336, K=4096)
    if want("quant_then_gemm_256x14336x4096"):
        M, N, K = 256, 14336, 4096
        x, gsx, _, _, wq, wsf, alpha = nv_inputs(M, N, K, 110, 112, b_std=0.02, outliers=True)
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        xsf = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        qfn = lambda: bs.quantize(x, "nvfp4", gs=gsx, q=xq, sf=xsf)
        gfn = lambda: bs.gemm(xq, xsf, wq, wsf, alpha, out=D)

        def both():
            qfn()
            gfn()
        qbytes = 2 * M * K + M * K // 2 + M * K // 16 + 4
        rows["quant_then_gemm_256x14336x4096"] = {
            "quant_cold": _rate(timer.run(qfn, cold=True), None, qbytes),
            "gemm_cold": _rate(timer.run(gfn, cold=True), 2.0 * M * N * K, _nv_bytes(M, N, K)),
            "pipeline_cold": _rate(timer.run(both, cold=True), 2.0 * M * N * K),
            "pipeline_warm": _rate(timer.run(both), 2.0 * M * N * K),
            "pipeline_graph": _rate(timer.graph(both), 2.0 * M * N * K)}

    # The page's 4-layer pipeline (back-to-back activation quantise + NVFP4 GEMM,
    # N = K = 7168, the same bf16 activation each layer): eager launches against
    # one HIP graph holding all 8 launches (the launch-gap-free analogue of the
    # page's PDL arm), and for up to four rows the fused quantise + GEMM (one
    # kernel per layer) in a graph.  The page's B300 SM103 numbers ride along as
    # context (none is printed for M = 4).
    if want("pipeline_4layer_7168"):
        N = K = 7168
        published = {1: (111.65, 107.10), 4: (None, None), 16: (112.42, 107.07), 64: (120.51, 115.65), 256: (120.83, 115.33),
                     1024: (151.52, 134.94), 2048: (250.27, 236.35), 4096: (432.38, 416.32)}
        b = bf16(synth.bf16_normal(180, (N, K), 0.02))
        gsb = bs.global_scale(b)
        bq, sfb = bs.quantize(b, "nvfp4", gs=gsb)
        del b
        res = {}
        for M in (1, 4, 16, 64, 256, 1024, 2048, 4096):
            a = bf16(synth.bf16_normal(181, (M, K)))
            gsa = torch.tensor([np.float32(0.5)], device=dev)  # a fixed global scale, as on the page
            aq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            asf = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            alpha = torch.tensor([np.float32(1.0)], device=dev)

            def layers():
                for _ in range(4):
                    bs.quantize(a, "nvfp4", gs=gsa, q=aq, sf=asf)
                    bs.gemm(aq, asf, bq, sfb, alpha, out=D)
            flops = 4 * 2.0 * M * N * K
            res[f"M={M}"] = {"eager": _rate(timer.run(layers, iters=10), flops),
                             "graph": _rate(timer.graph(layers, calls=5), flops),
                             "published_B300_no_pdl_us": published[M][0],
                             "published_B300_pdl_us": published[M][1]}
            if M <= 4:
                # the fused quantise + GEMM: one kernel per layer
                def fused_layers():
                    for _ in range(4):
                        bs.quantize_gemm(a, gsa, bq, sfb, alpha, out=D)
                fused_layers()
                ref = D.clone()
                layers()
                res[f"M={M}"]["fused_graph"] = _rate(timer.graph(fused_layers, calls=5), flops)
                res[f"M={M}"]["fused_matches_two_kernels"] = bool(torch.equal(D, ref))
            del a, aq, asf, D
        rows["pipeline_4layer_7168"] = res

    # a5: W4A16 at M=64 and M=1, N=4096, K=7168 (HBM roofline), and at M=4096
    # (the compute-bound regime, bf16 MFMA roofline)
    if want("w4a16_4096x7168"):
        res = {}
        N, K = 4096, 7168
        w = bf16(synth.bf16_normal(132, (N, K), 0.02))
        gw = bs.global_scale(w)
        wq, wsf = bs.quantize(w, "nvfp4", gs=gw)
        alpha = torch.tensor([np.float32(1.0) / np.float32(gw.cpu().numpy()[0])], device=dev)
        for M, seed in [(64, 130), (1, 131), (4096, 133)]:
            a = bf16(synth.bf16_normal(seed, (M, K)))
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fn = lambda: bs.w4a16_gemm(a, wq, wsf, alpha, out=D)
            nbytes = 2 * M * K + N * K // 2 + N * K // 16 + 4 + 2 * M * N
            res[f"M={M}"] = {"cold": _rate(timer.run(fn, cold=True), 2.0 * M * N * K, nbytes),
                             "warm": _rate(timer.run(fn), 2.0 * M * N * K, nbytes),
                             "algorithmic_bytes": nbytes}
            if M <= 64:
                res[f"M={M}"]["graph"] = _rate(timer.graph(fn), 2.0 * M * N * K, nbytes)
        rows["w4a16_4096x7168"] = res

    # W4A16 at the projection shapes of the W4A16 follow-up page (down: N=6656,
    # K=19968; up: N=19968, K=6656), M from weight streaming to compute bound;
    # "published_B_us" is the page's candidate arm on B300 (other hardware: context)
    if want("w4a16_projection_shapes"):
        published = {("down", 1): 54.176, ("down", 32): 54.497, ("down", 128): 55.089, ("down", 512): 117.489,
                     ("down", 2048): 289.411, ("down", 4096): 586.886, ("up", 1): 39.232, ("up", 32): 39.393,
                     ("up", 128): 45.792, ("up", 512): 103.473, ("up", 2048): 298.787, ("up", 4096): 599.638}
        res = {}
        for proj, N, K in [("down", 6656, 19968), ("up", 19968, 6656)]:
            w = bf16(synth.bf16_normal(170 if proj == "down" else 171, (N, K), 0.02))
            gw = bs.global_scale(w)
            wq, wsf = bs.quantize(w, "nvfp4", gs=gw)
            del w
            alpha = torch.tensor([np.float32(1.0) / np.float32(gw.cpu().numpy()[0])], device=dev)
            for M in (1, 32, 128, 512, 2048, 4096):
                a = bf16(synth.bf16_normal(172 + M, (M, K)))
                D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                fn = lambda: bs.w4a16_gemm(a, wq, wsf, alpha, out=D)
                nbytes = 2 * M * K + N * K // 2 + N * K // 16 + 4 + 2 * M * N
                r = _rate(timer.run(fn, iters=10, cold=True), 2.0 * M * N * K, nbytes)
                r["published_B_us"] = published[(proj, M)]
                res[f"{proj} M={M}"] = r
            del wq, wsf
        rows["w4a16_projection_shapes"] = res

    # a6: the MXFP4 form at the large workload shape (FP4 MFMA roofline)
    if want("mxfp4_gemm_4096x4096x7168"):
        M, N, K = 4096, 4096, 7168
        a = bf16(synth.bf16_normal(120, (M, K)))
        b = bf16(synth.bf16_normal(121, (N, K)))
        aq, sfa = bs.quantize(a, "mxfp4")
        bq, sfb = bs.quantize(b, "mxfp4")
        del a, b
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fn = lambda: bs.gemm(aq, sfa, bq, sfb, None, fmt="mxfp4", out=D)
        nbytes = M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + 2 * M * N
        rows["mxfp4_gemm_4096x4096x7168"] = {
            "warm": _rate(timer.run(fn), 2.0 * M * N * K, nbytes),
            "cold": _rate(timer.run(fn, iters=10, cold=True), 2.0 * M * N * K, nbytes),
            "bound": "mfma (fp4)", "peak_tflops": PEAK["fp4"]}

    # a2, a7-a10: the MXFP4 MoE layer (4096 tokens, hidden 2048, 128 experts, top-8, I=768)
    if want("moe_mxfp4_4096x2048_e128_top8"):
        T, H, I, E, topk = 4096, 2048, 768, 128, 8
        x = bf16(synth.bf16_normal(140, (T, H)))
        ids_np, w_np = synth.routing(141, T, E, topk)
        ids = torch.from_numpy(ids_np).to(dev)
        tw = torch.from_numpy(w_np.reshape(-1)).to(dev)
        w13 = bf16(synth.bf16_normal(142, (E * 2 * I, H), 0.02))
        W13, W13sf = bs.quantize(w13, "mxfp4")
        del w13
        w2 = bf16(synth.bf16_normal(143, (E * H, I), 0.02))
        W2, W2sf = bs.quantize(w2, "mxfp4")
        del w2
        W13, W13sf = W13.view(E, 2 * I, H // 2), W13sf.view(E, 2 * I, H // 32)
        W2, W2sf = W2.view(E, H, I // 2), W2sf.view(E, H, I // 32)
        ROW_INPUTS["moe_mxfp4"] = (x, ids, tw, W13, W13sf, W2, W2sf)
        R = T * topk
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        sids = torch.empty(R, dtype=torch.int32, device=dev)
        stok = torch.empty(R, dtype=torch.int32, device=dev)
        xq = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
        xsf = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        aq = torch.empty((R, I // 2), dtype=torch.uint8, device=dev)
        asf = torch.empty((R, I // 32), dtype=torch.uint8, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        lib = bs.load()
        import ctypes
        ws_bytes = lib.mxfp4_moe_grouped_gemm_workspace_size(R, E, H, I, bs.MOE_WEIGHTED_COMBINE, T)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        from block_scaled_fp4_e2m1_amd import binding as B

        def prep():
            B._check(lib.fp4_moe_prep(B._p(ids), T, topk, E, B._p(offs), B._p(sids), B._p(stok), None, 0,
                                      B._stream(dev)), "prep")

        def equant():  # each token once; the gate_up GEMM reads rows by token
            bs.quantize(x, "mxfp4", q=xq, sf=xsf)

        a1 = B.MoeEpilogueArgs(out_q=aq.data_ptr(), out_sf=asf.data_ptr())
        a2 = B.MoeEpilogueArgs(out=out.data_ptr(), sorted_ids=sids.data_ptr(), topk_weights=tw.data_ptr(),
                               num_tokens=T, topk=topk)

        def gemm1():
            B._check(lib.mxfp4_moe_grouped_gemm(B._p(xq), B._p(xsf), T, B._p(stok), B._p(offs), E, R, B._p(W13),
                                                B._p(W13sf), 2 * I, H, bs.MOE_SILU_MUL_QUANT, ctypes.byref(a1),
                                                None, 0, B._stream(dev)), "gemm1")

        def gemm2():
            B._check(lib.mxfp4_moe_grouped_gemm(B._p(aq), B._p(asf), R, None, B._p(offs), E, R, B._p(W2),
                                                B._p(W2sf), H, I, bs.MOE_WEIGHTED_COMBINE, ctypes.byref(a2),
                                                B._p(ws), ws_bytes, B._stream(dev)), "gemm2")

        def layer():
            prep()
            equant()
            gemm1()
            gemm2()
        wbytes = W13.numel() + W13sf.numel() + W2.numel() + W2sf.numel()
        # weights + x read + out written + quantised x written/read + act codes written/read
        nbytes = wbytes + 2 * T * H * 2 + 2 * (xq.numel() + xsf.numel()) + 2 * (aq.numel() + asf.numel())
        flops = 2.0 * R * (2 * I) * H + 2.0 * R * H * I
        layer()
        ref = out.clone()
        rows["moe_mxfp4_4096x2048_e128_top8"] = {
            "layer_cold": _rate(timer.run(layer, iters=10, cold=True), flops, nbytes),
            "layer_warm": _rate(timer.run(layer, iters=10), flops, nbytes),
            "layer_graph": _rate(timer.graph(layer, calls=3), flops, nbytes),
            "graph_matches_eager": bool(torch.equal(out, ref)),
            "stages_cold_us": {"prep": timer.run(prep, cold=True)["median_us"],
                               "experts_quant": timer.run(equant, cold=True)["median_us"],
                               "gate_up_silu_quant": timer.run(gemm1, cold=True)["median_us"],
                               "down_combine": timer.run(gemm2, cold=True)["median_us"]},
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "bound": "hbm (weights are 83% of the bytes)"}

    # f2: the NVFP4 MoE layer at the same shape (per-expert global scales and
    # alphas; every routed row quantised with its expert's scale)
    if want("moe_nvfp4_4096x2048_e128_top8"):
        T, H, I, E, topk = 4096, 2048, 768, 128, 8
        R = T * topk
        x = bf16(synth.bf16_normal(240, (T, H)))
        ids_np, w_np = synth.routing(241, T, E, topk)
        ids = torch.from_numpy(ids_np).to(dev)
        tw = torch.from_numpy(w_np.reshape(-1)).to(dev)
        w13 = bf16(synth.bf16_normal(242, (E * 2 * I, H), 0.02))
        g13 = bs.global_scale(w13)
        W13, W13sf = bs.quantize(w13, "nvfp4", gs=g13)
        del w13
        w2 = bf16(synth.bf16_normal(243, (E * H, I), 0.02))
        g2 = bs.global_scale(w2)
        W2, W2sf = bs.quantize(w2, "nvfp4", gs=g2)
        del w2
        W13, W13sf = W13.view(E, 2 * I, H // 2), W13sf.view(E, 2 * I, H // 16)
        W2, W2sf = W2.view(E, H, I // 2), W2sf.view(E, H, I // 16)
        offs, sids, stok = bs.moe_prep(ids, E)
        gs1 = bs.global_scale(x).expand(E).contiguous()
        alpha1 = 1.0 / (gs1 * g13)
        xq, xsf = bs.nvfp4_experts_quantize(x, offs, gs1, row_map=stok)
        # act scale calibration (setup): the gate_up rows' SiLU-gated amax
        h1 = bs.nvfp4_moe_grouped_gemm(xq, xsf, offs, W13, W13sf, alpha1, bs.MOE_STORE_BF16).float()
        act = (torch.nn.functional.silu(h1[:, :I]) * h1[:, I:]).to(torch.bfloat16)
        gs2 = bs.global_scale(act).expand(E).contiguous()
        del h1, act
        alpha2 = 1.0 / (gs2 * g2)
        aq = torch.empty((R, I // 2), dtype=torch.uint8, device=dev)
        asf = torch.empty((R, I // 16), dtype=torch.uint8, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        lib = bs.load()
        import ctypes
        from block_scaled_fp4_e2m1_amd import binding as B
        ws_bytes = lib.nvfp4_moe_grouped_gemm_workspace_size(R, E, H, I, bs.MOE_WEIGHTED_COMBINE, T)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def prep():
            B._check(lib.fp4_moe_prep(B._p(ids), T, topk, E, B._p(offs), B._p(sids), B._p(stok), None, 0,
                                      B._stream(dev)), "prep")

        def equant():
            B._check(lib.nvfp4_experts_quantize(B._p(x), T, H, B._p(stok), B._p(offs), E, B._p(gs1), R,
                                                B._p(xq), B._p(xsf), B._stream(dev)), "equant")

        a1 = B.MoeEpilogueArgs(out_q=aq.data_ptr(), out_sf=asf.data_ptr(), out_gs=gs2.data_ptr())
        a2 = B.MoeEpilogueArgs(out=out.data_ptr(), sorted_ids=sids.data_ptr(), topk_weights=tw.data_ptr(),
                               num_tokens=T, topk=topk)

        def gemm1():
            B._check(lib.nvfp4_moe_grouped_gemm(B._p(xq), B._p(xsf), B._p(offs), E, R, B._p(W13), B._p(W13sf),
                                                B._p(alpha1), 2 * I, H, bs.MOE_SILU_MUL_QUANT, ctypes.byref(a1),
                                                None, 0, B._stream(dev)), "gemm1")

        def gemm2():
            B._check(lib.nvfp4_moe_grouped_gemm(B._p(aq), B._p(asf), B._p(offs), E, R, B._p(W2), B._p(W2sf),
                                                B._p(alpha2), H, I, bs.MOE_WEIGHTED_COMBINE, ctypes.byref(a2),
                                                B._p(ws), ws_bytes, B._stream(dev)), "gemm2")

        def layer():
            prep()
            equant()
            gemm1()
            gemm2()
        wbytes = W13.numel() + W13sf.numel() + W2.numel() + W2sf.numel()
        # weights + x read + out written + quantised rows written/read + act codes written/read
        nbytes = wbytes + 2 * T * H * 2 + 2 * (xq.numel() + xsf.numel()) + 2 * (aq.numel() + asf.numel())
        flops = 2.0 * R * (2 * I) * H + 2.0 * R * H * I
        layer()
        ref = out.clone()
        rows["moe_nvfp4_4096x2048_e128_top8"] = {
            "layer_cold": _rate(timer.run(layer, iters=10, cold=True), flops, nbytes),
            "layer_warm": _rate(timer.run(layer, iters=10), flops, nbytes),
            "layer_graph": _rate(timer.graph(layer, calls=3), flops, nbytes),
            "graph_matches_eager": bool(torch.equal(out, ref)),
            "stages_cold_us": {"prep": timer.run(prep, cold=True)["median_us"],
                               "experts_quant": timer.run(equant, cold=True)["median_us"],
                               "gate_up_silu_quant": timer.run(gemm1, cold=True)["median_us"],
                               "down_combine": timer.run(gemm2, cold=True)["median_us"]},
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "bound": "mfma (fp16 on the exact dequantised values)", "peak_tflops": PEAK["f16"]}
    return rows


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_of_3(fn):
    """One untimed warm run, then the median wall time of three runs."""
    fn()
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        r = fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)), r


# tensors of the MoE row kept for the oracle's timing (host copies are made there)
ROW_INPUTS = {}


def cpu_baseline(torch, bs, synth, bf16, inputs):
    """The oracle on this host, timed as: one warm run, then the median of three.

    Headline (value): the float64 GEMM oracle on the whole 4096 x 4096 x 7168
    workload with the BLAS pool on every core (it is also checked against the
    GPU output element by element).  Beside it: the same GEMM on one core (a
    256-row sample), the 16 x 4096 x 7168 GEMM, the NVFP4 quantiser of the
    256 x 4096 activations (numpy element-wise code runs on one core), and the
    MoE layer on a 128-token sample of the 4096-token workload (all 128
    experts, top-8) with the workload's quantised weights."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import gemm as OG
    from oracle import moe as OM
    from oracle import quant as OQ
    from oracle import tolerance as TOL

    aq, sfa, bq, sfb, alpha, D = inputs
    A, SA, B, SB = aq.cpu().numpy(), sfa.cpu().numpy(), bq.cpu().numpy(), sfb.cpu().numpy()
    al = float(alpha.cpu().numpy()[0])
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    secs, ref = _median_of_3(lambda: OG.nvfp4_gemm(A, SA, B, SB, al))
    flops = 2.0 * A.shape[0] * B.shape[0] * B.shape[1] * 2
    got = D.view(torch.int16).cpu().numpy().view(np.uint16)
    ok, worst, nbad = TOL.check_bf16(got, ref)
    per = {}

    rows1 = slice(0, 256)
    with threadpool_limits(limits=1):
        t1, _ = _median_of_3(lambda: OG.nvfp4_gemm(A[rows1], SA[rows1], B, SB, al))
    per["nvfp4_gemm_4096x4096x7168_1core"] = {
        "seconds": round(t1, 4), "tflops": round(2.0 * 256 * B.shape[0] * B.shape[1] * 2 / t1 / 1e12, 6),
        "cores": 1, "sample": "rows 0..255 of A, all 4096 columns, K=7168"}

    # config 0: 16 x 4096 x 7168 (inputs quantised on the GPU, seeds 100 / 101)
    a0 = bf16(synth.bf16_normal(100, (16, 7168)))
    b0 = bf16(synth.bf16_normal(101, (4096, 7168)))
    g0a, g0b = bs.global_scale(a0), bs.global_scale(b0)
    q0a, s0a = bs.quantize(a0, "nvfp4", gs=g0a)
    q0b, s0b = bs.quantize(b0, "nvfp4", gs=g0b)
    g0 = torch.cat([g0a, g0b]).cpu().numpy()
    al0 = float(np.float32(1.0) / np.float32(g0[0] * g0[1]))
    H0 = [t.cpu().numpy() for t in (q0a, s0a, q0b, s0b)]
    t0s, _ = _median_of_3(lambda: OG.nvfp4_gemm(*H0, al0))
    per["nvfp4_gemm_16x4096x7168"] = {"seconds": round(t0s, 4), "cores": int(threads),
                                      "tflops": round(2.0 * 16 * 4096 * 7168 / t0s / 1e12, 6),
                                      "gbs": round(_nv_bytes(16, 4096, 7168) / t0s / 1e9, 3),
                                      "sample": "the whole workload"}

    # config 1's producer: the NVFP4 quantiser on 256 x 4096 bf16 with outliers
    x1 = synth.bf16_normal_with_outliers(110, 1110, (256, 4096))
    gs1 = OQ.global_scale(x1)
    with threadpool_limits(limits=1):
        tq, _ = _median_of_3(lambda: OQ.nvfp4_quantize(x1, gs1))
    per["nvfp4_quantize_256x4096"] = {
        "seconds": round(tq, 5), "cores": 1, "gbs": round((2 * 256 * 4096) / tq / 1e9, 4),
        "sample": "the whole workload; numpy element-wise code runs on one core, so one core and all cores "
                  "are the same run"}

    # config 4: the MXFP4 MoE layer on a 128-token sample
    moe = ROW_INPUTS.get("moe_mxfp4")
    if moe is not None:
        Ts = 128
        x, ids, w, W13, W13sf, W2, W2sf = moe
        xs = x[:Ts].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        ids_s, w_s = ids[:Ts].cpu().numpy(), w.view(-1, ids.shape[1])[:Ts].cpu().numpy()
        Wh = [t.cpu().numpy() for t in (W13, W13sf, W2, W2sf)]
        tm, _ = _median_of_3(lambda: OM.moe_layer(xs, ids_s, w_s, *Wh))
        E, I2, Hh = W13.shape
        R = Ts * ids.shape[1]
        mflops = 2.0 * R * I2 * (Hh * 2) + 2.0 * R * (Hh * 2) * (I2 // 2)
        per["moe_mxfp4_4096x2048_e128_top8"] = {
            "seconds": round(tm, 3), "cores": int(threads), "tflops": round(mflops / tm / 1e12, 6),
            "sample": f"tokens 0..{Ts - 1} of 4096 (top-8 of 128 experts, {R} routed rows), every stage"}

    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(secs, 3), "timing": "median of 3 after one warm run",
            "cpu_model": _cpu_model(), "nproc": nproc,
            "sample": "full workload: 4096 rows x 4096 columns x K=7168 "
                      "(exact float64 dequant + float64 matmul + bf16 rounding)",
            "parity_on_sample": {"ok": ok, "worst_ratio": round(worst, 4), "n_bad": nbad},
            "per_config": per}


if __name__ == "__main__":
    main()
