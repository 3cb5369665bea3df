#!/usr/bin/env python3
"""Throughput of the HLA-2 forward hot path on one MI355X.

One step = one whole forward pass (segment summaries -> up-sweep of the
exclusive Blelloch scan -> per-segment prefix and chunked forward) over one
batch of the headline workload: ratio-
normalised HLA-2, B=8, H=16, n=4096, d=dv=64, bf16 inputs and output, fp32
state, q, k ~ U[0,1)/sqrt(d), v ~ N(0,1), seeded.  Inputs are resident in
HBM before the timed region.  Prints ONE JSON line on stdout; progress goes
to stderr.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Timing: first untimed steps for at least --settle-ms (300 ms: the GPU's
clocks ramp over the first few hundred ms of load, and steps timed before
that run up to 15% slower), then W warm-up steps; then
K steps between two synchronisations, one library call per step,
with HIP events only at the two ends, on the stream the library launches on
(torch's current stream): that gives ms_per_step and the throughput.  A
second pass of K steps brackets every stage with events on the same stream,
which splits the step by stage (the markers add small gaps, so that pass is
not the throughput).  A third pass launches each stage K times back to back
between two events: the per-kernel times, which the roofline figure uses;
the largest stage is then launched K times more, each launch after a read
of a 1 GiB buffer outside its events (roofline.cold: no Infinity Cache hits
on its inputs; a read rather than a write, whose dirty lines would drain to
HBM during the timed launch).  Then: K steps with an
event between consecutive steps (median, p10, p90 per step); K cold steps,
each after the same 1 GiB read (more than the Infinity Cache);
and K replays of the step captured in a HIP graph.  Decode is timed as the
mean over 1024 plain calls and over replays of 64 captured steps (a spread
per call would time the host: a 3.5 us step is shorter than one submission).  Then the
backward (HLA-2 gradients at the same shape, and the ratio gradients on the
benchmark's own inputs) and the third-order forward, each as calls between two
events.  The CPU baseline is the fp64
oracle on the same inputs (all heads), on the host's cores; its output is
compared with the benchmarked GPU output, every element (parity_rel_l2).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3
METRIC = "HLA-2 forward tokens/sec (B·H·n/s) + % MFMA peak, n=4096 d=64 bf16"
CSRC = os.path.join(ROOT, "causal_streaming_scans_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of every kernel and library source: stored counter figures are used
    only while it matches the hash they were taken on."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "hla2_forward_counters.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or rec.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def trace_summary(trace_csv: str, bench_json: str) -> None:
    """Per-pass kernel durations from a rocprofv3 kernel trace of one bench.py
    run (`--kernel-trace`, csv) and that run's JSON line: each stage kernel's
    dispatches in launch order, past the settle and warm-up steps, split into
    the timed pass, the stage pass and the back-to-back pass (K each)."""
    import csv
    import statistics
    with open(bench_json) as fh:
        rec = json.loads(fh.read().strip().splitlines()[-1])
    skip, K = rec["settle"]["steps"] + rec["warmup"], rec["steps"]
    with open(trace_csv) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
    per = {}
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"settle + warm-up steps skipped: {skip}; K = {K}")
    # backward leg: its last `backward_steps` passes of la_ launches, by
    # position within a pass (the pass order of hla_backward)
    bwd = [r for r in rows if is_la_kernel(r["Kernel_Name"])]
    nb = (rec.get("backward") or {}).get("launches_per_step", 0)
    Kb = (rec.get("backward") or {}).get("steps", 0)
    for name, us in per.items():
        if is_la_kernel(name) or not is_stage_kernel(name):
            continue
        parts = {"timed": us[skip:skip + K], "stages": us[skip + K:skip + 2 * K],
                 "back-to-back": us[skip + 2 * K:skip + 3 * K]}
        print(name)
        for label, v in parts.items():
            if v:
                print(f"    {label:13s} n={len(v):5d} avg {statistics.fmean(v):8.2f} us"
                      f"  min {min(v):8.2f}  max {max(v):8.2f}")
    if nb and Kb and len(bwd) >= nb * (10 + Kb):
        # the HLA-2 leg: 10 untimed calls, then Kb timed ones (the ratio leg follows)
        last = bwd[10 * nb:(10 + Kb) * nb]
        print(f"backward: the {Kb} timed HLA-2 backward calls, {nb} launches each")
        total = 0.0
        for i in range(nb):
            v = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in last[i::nb]]
            total += statistics.fmean(v)
            print(f"    {i:2d} {kernel_key(last[i]['Kernel_Name']):20s} grid {last[i]['Grid_Size_X']:>8s}"
                  f"  avg {statistics.fmean(v):8.2f} us")
        print(f"    sum of averages {total:8.2f} us")


def is_la_kernel(name: str) -> bool:
    """A first-order linear-attention kernel (backward passes, third order's
    Y), not an AHLA kernel whose name also contains "la_"."""
    import re
    return re.search(r"(?<![a-z])la_(summary|forward)_kernel", name) is not None


_STAGE_RE = r"(hla2_|ahla_|la_)?(summary|up_sweep|forward)(_pipe)?_kernel"


def is_stage_kernel(name: str) -> bool:
    """A kernel of the forward path's three stages (or a la_ pass kernel)."""
    import re
    return re.search(_STAGE_RE, name) is not None


def kernel_key(name: str) -> str:
    """Short key of a stage kernel from its (mangled or demangled) name: the
    forward path's hla2_/ahla_ kernels and the up-sweep, and the backward's
    la_ kernels, whose two-slot (SYM) instances get a _sym suffix.  The
    pipelined HLA-2 forward kernel is stage 3's kernel: hla2_forward_kernel.
    The stage-3 forms that also write their first pass's rows (hla_forward_z;
    the last template flag) get a _z suffix."""
    import re
    m = re.search(_STAGE_RE, name)
    key = (m.group(1) or "") + m.group(2) + "_kernel"
    if key in ("hla2_forward_kernel", "ahla_forward_kernel"):
        mz = re.search(r"Lb([01])EEEv", name) or re.search(r"(true|false)>\(", name)
        if mz and mz.group(1) in ("1", "true"):
            key = key[:-len("_kernel")] + "_z_kernel"
    if key.startswith("la_"):
        # template flags (SYM, DUAL): mangled ...Lb<0|1>ELb<0|1>E, or demangled
        mm = re.search(r"Lb([01])ELb([01])E", name)
        md = re.search(r"(true|false), (true|false)>", name)
        flags = (mm.group(1) == "1", mm.group(2) == "1") if mm else \
            ((md.group(1) == "true", md.group(2) == "true") if md else (False, False))
        if flags[0]:
            key += "_sym"
        if flags[1]:
            key += "_dual"
        if "<float" in name or re.search(r"kernelIf", name):
            key += "_f32"
    return key


def counters_summary(fetch_csv: str, write_csv: str) -> None:
    """HBM bytes per launch of each stage kernel from two `rocprofv3 --pmc` runs
    of bench.py with --copy-calibration-mib (FETCH_SIZE, then WRITE_SIZE; csv).
    Each counter's KiB per dispatch is scaled by what it reads for the torch.neg
    copy of known size.  Prints the JSON record bench.py reads back."""
    import csv
    import re
    import statistics

    def per_kernel(path, counter):
        per = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        out = {}
        for (name, _), val in per.items():
            out.setdefault(name, []).append(val)
        return {name: statistics.fmean(v) for name, v in out.items()}

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    neg = [n for n in fetch if "neg" in n]
    if not neg:
        raise SystemExit("no torch.neg calibration dispatches in the counter csv")
    cal_f, cal_w = fetch[neg[0]], write[[n for n in write if "neg" in n][0]]
    mib = round(cal_w / 1024)            # KiB written by the copy -> its size in MiB
    fs, ws = mib * 1024 / cal_f, mib * 1024 / cal_w
    rec = {"source_hash": kernel_source_hash(),
           "workload": "HLA-2 ratio B=8 H=16 n=4096 d=dv=64 bf16, default launch configuration",
           "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
           "copy_calibration": {"kernel": f"torch.neg over {mib} MiB bf16 ({mib} MiB read, "
                                          f"{mib} MiB written)",
                                "FETCH_SIZE_KiB": round(cal_f, 1), "WRITE_SIZE_KiB": round(cal_w, 1)}}
    def entry(name):
        fb, wb = fetch[name] * 1024 * fs, write[name] * 1024 * ws
        return {"FETCH_SIZE_KiB": round(fetch[name], 1), "WRITE_SIZE_KiB": round(write[name], 1),
                "fetch_bytes": int(fb), "write_bytes": int(wb), "hbm_bytes_per_launch": int(fb + wb)}

    for short in ("summary_kernel", "up_sweep_kernel", "forward_kernel"):
        names = [n for n in fetch if is_stage_kernel(n) and kernel_key(n).endswith(short)
                 and n in write]
        for name in names:
            rec[kernel_key(name)] = entry(name)
    # the decode step (AHLA, 32 heads, d = 64) when the runs timed it
    dec = [n for n in fetch if "ahla_step_sliced_kernel" in n and n in write]
    if dec:
        rec["ahla_step_sliced_kernel"] = entry(dec[0])
    print(json.dumps(rec, indent=1))


def short_kernel_name(name: str) -> str:
    """hla::<kernel><template arguments> from a mangled or demangled kernel name,
    e.g. hla2_forward_kernel<bf16,64,64,64,0>."""
    import re
    m = re.search(r"_ZN3hla\d+(\w+?)I(.*?)EEvNS_", name)
    if m:
        parts = []
        for tok in re.finditer(r"DF16b|Lb[01]|Li\d+|f(?=L|E)", m.group(2)):
            t = tok.group(0)
            parts.append("bf16" if t == "DF16b" else "float" if t == "f" else
                         t[2:] if t.startswith("Li") else t[2:])
        return f"{m.group(1)}<{','.join(parts)}>"
    m = re.search(r"hla::(\w+)", name)
    return m.group(1) if m else name[:80]


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
SIMD_COUNT = 256 * 4     # MI355X: 256 compute units of 4 SIMDs
XCD_COUNT = 8            # GRBM_GUI_ACTIVE arrives summed over the 8 XCDs
NOMINAL_CLOCK_HZ = 2.4e9  # MI355X peak engine clock


def mfma_summary(csv_path: str) -> None:
    """Counter-measured matrix-core use per kernel and launch shape, from one
    `rocprofv3 --pmc` run with the four MFMA_COUNTERS (csv).  Per dispatch:
    MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES (summed over every SIMD) /
    (GRBM_GUI_ACTIVE / XCD_COUNT x SIMD_COUNT) (rocprof's MfmaUtil), and
    the same over the dispatch's timestamp span at 2.4 GHz (short dispatches
    count more GUI_ACTIVE cycles than their span, so the first reads low); executed bf16 / fp32 MFMA flops =
    SQ_INSTS_VALU_MFMA_MOPS_* x 512; TFLOP/s over the dispatch's own
    timestamps.  GRBM_GUI_ACTIVE arrives summed over the XCDs, so one XCD's
    busy cycles (the dispatch's length in GPU clocks) are that over XCD_COUNT.
    Averages over the dispatches of each (kernel, grid) pair;
    prints one JSON record."""
    import csv
    import statistics

    per = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            key = (r["Kernel_Name"], int(r["Grid_Size"]), r["Dispatch_Id"])
            d = per.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            c, val = r["Counter_Name"], float(r["Counter_Value"])
            # GRBM_GUI_ACTIVE may be listed twice for one dispatch (same value)
            d[c] = max(d.get(c, 0.0), val) if c == "GRBM_GUI_ACTIVE" else d.get(c, 0.0) + val
    groups = {}
    for (name, grid, _), d in per.items():
        if not all(c in d for c in MFMA_COUNTERS):
            continue
        groups.setdefault((name, grid), []).append(d)
    rows = []
    for (name, grid), ds in sorted(groups.items(), key=lambda kv: -len(kv[1])):
        mean = lambda f: statistics.fmean(f(d) for d in ds)
        busy = mean(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"]
                    / (d["GRBM_GUI_ACTIVE"] / XCD_COUNT * SIMD_COUNT))
        mhz = mean(lambda d: d["GRBM_GUI_ACTIVE"] / XCD_COUNT / (d["ns"] * 1e-3))
        busy_ts = mean(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"]
                       / (SIMD_COUNT * d["ns"] * 1e-9 * NOMINAL_CLOCK_HZ))
        fl_bf16 = mean(lambda d: d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512)
        fl_f32 = mean(lambda d: d["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512)
        us = mean(lambda d: d["ns"]) * 1e-3
        if fl_bf16 + fl_f32 == 0:
            continue
        rows.append({"kernel": short_kernel_name(name), "grid_threads": grid, "dispatches": len(ds),
                     "us": round(us, 2), "gpu_clock_mhz": round(mhz),
                     "mfma_busy_pct": round(100 * busy, 2),
                     "mfma_busy_pct_of_span": round(100 * busy_ts, 2),
                     "bf16_mfma_gflop": round(fl_bf16 * 1e-9, 3),
                     "f32_mfma_gflop": round(fl_f32 * 1e-9, 3),
                     "bf16_tflops": round(fl_bf16 / (us * 1e-6) * 1e-12, 1) if us > 0 else None,
                     "bf16_peak_frac": round(fl_bf16 / (us * 1e-6) * 1e-12 / BF16_MFMA_PEAK_TFLOPS, 4)
                     if us > 0 else None})
    print(json.dumps({"source_hash": kernel_source_hash(), "counters": list(MFMA_COUNTERS),
                      "kernels": rows}, indent=1))


def all_configs(args, hla, I, torch, dev):
    """Forward time of every named workload in its default launch
    configuration (each one library call between two events, after a settle
    phase of --settle-ms); one JSON line.  Only the forward is timed: the AHLA workload's
    decode tokens are timed by the default run."""
    rows = []
    for key, w in I.WORKLOADS.items():
        x = I.workload_inputs(key, decode_tokens=0)
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        shp = (w.B, w.H, w.n, w.d)
        q, k, v = (torch.from_numpy(x[n]).reshape(shp).to(dev, tdt).contiguous() for n in "qkv")
        gamma = x["gamma"]
        del x
        plan = hla.ForwardPlan(q, k, v, variant=w.variant, gamma=gamma, chunk=w.chunk)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        settle = 0.0
        while settle < args.settle_ms:
            e0.record()
            for _ in range(20):
                plan.run()
            e1.record()
            torch.cuda.synchronize()
            settle += e0.elapsed_time(e1)
        K = max(20, args.steps // 10)
        e0.record()
        for _ in range(K):
            plan.run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        tokens = w.B * w.H * w.n
        esz = 2 if w.dtype == "bf16" else 4
        lean = tokens * (2 * w.d + 2 * w.dv) * esz
        rows.append({"workload": w.name, "timed": "forward", "variant": w.variant, "chunk": w.chunk,
                     "seg_chunks": hla.default_seg_chunks(w.variant, w.B, w.H, w.n, w.d, w.chunk),
                     "ms": round(ms, 5), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
                     "lean_hbm_frac": round(lean / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        log(f"[bench] {w.name}: {ms:.4f} ms, {tokens / (ms * 1e-3) / 1e9:.3f} G tokens/s")
        del q, k, v, plan
    print(json.dumps({"forward_per_workload": rows}), flush=True)


def flops_per_token(c, d, dv):
    # dense products of the chunked method per token: scores 2cd, Q S0 2d^2,
    # L K 2cd, Q Z^T 2cd, P V 2c dv, Q W0 2d dv, S update 2d^2, W update 2d dv
    return 6 * c * d + 2 * c * dv + 4 * d * d + 4 * d * dv


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for at least this long before the warm-up steps, so "
                         "the GPU is at its steady clocks when timing starts")
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--seg-chunks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--backward-steps", type=int, default=200,
                    help="time this many hla_backward calls (HLA-2 and ratio gradients at the "
                         "benchmark shape) and third-order forwards; 0 skips these legs")
    ap.add_argument("--backward-seg-chunks", type=int, default=0,
                    help="chunks per segment of the backward passes (0 = the library default)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle over the workload until this much wall time")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the workload, run a plain elementwise copy (torch.neg) of "
                         "this many MiB in and out, whose HBM counters scale the kernel's")
    ap.add_argument("--all-configs", action="store_true",
                    help="time the forward of every named workload (and the AHLA decode), "
                         "print one JSON line, then exit")
    ap.add_argument("--print-source-hash", action="store_true")
    ap.add_argument("--counters-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM-traffic record from two rocprofv3 --pmc counter csv "
                         "files of a bench.py run (FETCH_SIZE, then WRITE_SIZE), then exit")
    ap.add_argument("--mfma-summary", metavar="PMC_CSV",
                    help="per-kernel MFMA busy %% and executed MFMA flops from a rocprofv3 --pmc "
                         "run with the counters " + " ".join(MFMA_COUNTERS))
    ap.add_argument("--trace-summary", nargs=2, metavar=("KERNEL_TRACE_CSV", "BENCH_JSON"),
                    help="print per-pass kernel durations from a rocprofv3 kernel trace of a "
                         "bench.py run and that run's JSON line, then exit")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.counters_summary:
        counters_summary(*args.counters_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.print_source_hash:
        print(kernel_source_hash())
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_streaming_scans_amd as hla
    from causal_streaming_scans_amd import inputs as I

    hla.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.all_configs:
        all_configs(args, hla, I, torch, dev)
        return
    if args.copy_calibration_mib > 0:
        nel = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.ones(nel, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] copy calibration: 3 x torch.neg over {args.copy_calibration_mib} MiB")
    w = I.WORKLOADS["ratio_n4096"]
    B, H, n, d, dv, chunk = w.B, w.H, w.n, w.d, w.dv, args.chunk
    variant = w.variant
    seg = args.seg_chunks or hla.default_seg_chunks(variant, B, H, n, d, chunk)
    nseg = -(-n // (chunk * seg))
    log(f"[bench] workload {w.name}: chunk {chunk}, {seg} chunks/segment, {nseg} segments")

    x = I.workload_inputs("ratio_n4096")

    def to_dev(a, shape):
        return torch.from_numpy(a).reshape(shape).to(torch.bfloat16).to(dev).contiguous()

    q = to_dev(x["q"], (B, H, n, d))
    k = to_dev(x["k"], (B, H, n, d))
    v = to_dev(x["v"], (B, H, n, dv))
    o = torch.empty((B, H, n, dv), dtype=torch.bfloat16, device=dev)
    ws_bytes = hla.workspace_bytes(variant, B, H, n, d, dv, chunk, seg)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    # arguments marshalled once: each stage below is one library call
    plan = hla.ForwardPlan(q, k, v, variant=variant, chunk=chunk, seg_chunks=seg, out=o,
                           workspace=ws, staged=True)

    def step():
        plan.run()

    # ---- settle: untimed steps until the GPU has run them for settle_ms (its
    # clocks ramp over the first few hundred ms of load), then W warm-up steps
    settle_steps, settle_ms = 0, 0.0
    e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while settle_ms < args.settle_ms and settle_steps < 100000:
        e_a.record()
        for _ in range(100):
            step()
        e_b.record()
        torch.cuda.synchronize()
        settle_ms += e_a.elapsed_time(e_b)
        settle_steps += 100
    log(f"[bench] settle: {settle_steps} untimed steps, {settle_ms:.0f} ms")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, one library call each, bracketed by
    # events only at its two ends
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(K):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / K

    # ---- the stages of K more steps, each bracketed by events on the same
    # stream (the markers add small gaps, so this pass only splits the time)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        ev[s][0].record()
        for stage in (1, 2, 3):
            plan.stage(stage)
            ev[s][stage].record()
    torch.cuda.synchronize()
    stage_ms = [float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)]))
                for i in range(3)]
    # ---- per-kernel time: each stage launched K times back to back between two
    # events (each stage is idempotent given the previous one's output), so no
    # dependency gap of the step sits inside the figure
    kern_ms = []
    for stage in (1, 2, 3):
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(K):
            plan.stage(stage)
        t_end.record()
        torch.cuda.synchronize()
        kern_ms.append(t_start.elapsed_time(t_end) / K)
    # ---- cold launches: before each, a 1 GiB buffer (more than the 256 MB
    # Infinity Cache) is read, outside the timed events, so the launch finds
    # none of its inputs in that cache.  A read, not a write: a written
    # buffer leaves dirty lines whose write-back to HBM would run during the
    # timed launch and be charged to it
    scrub = torch.zeros(1 << 28, dtype=torch.float32, device=dev)

    def scrub_caches():
        scrub.sum()

    # the largest stage again, each launch cold: back-to-back launches find
    # part of their inputs in the Infinity Cache, these do not
    dom = int(np.argmax(kern_ms))
    evk = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        scrub_caches()
        evk[s][0].record()
        plan.stage(dom + 1)
        evk[s][1].record()
    torch.cuda.synchronize()
    kern_cold_ms = float(np.median([a.elapsed_time(b) for a, b in evk]))
    tokens = B * H * n
    tok_s = tokens / (ms_per_step * 1e-3)
    log(f"[bench] {ms_per_step:.4f} ms/step, {tok_s / 1e9:.3f} G tokens/s; stages (ms) "
        f"summary {stage_ms[0]:.4f} up-sweep {stage_ms[1]:.4f} forward {stage_ms[2]:.4f}; "
        f"back-to-back launches (ms) {kern_ms[0]:.4f} {kern_ms[1]:.4f} {kern_ms[2]:.4f}; "
        f"stage {dom + 1} after a cache scrub (median ms) {kern_cold_ms:.4f}")

    def pct(a):
        a = np.asarray(a, np.float64)
        return {"median_ms": round(float(np.median(a)), 5), "p10_ms": round(float(np.percentile(a, 10)), 5),
                "p90_ms": round(float(np.percentile(a, 90)), 5)}

    # ---- per-step spread: K more steps with an event between consecutive steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for s in range(K):
        step()
        evs[s + 1].record()
    torch.cuda.synchronize()
    warm = pct([evs[i].elapsed_time(evs[i + 1]) for i in range(K)])

    # ---- cold steps: the 1 GiB scrub buffer is read before each step,
    # outside the step's own events
    evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        scrub_caches()
        evc[s][0].record()
        step()
        evc[s][1].record()
    torch.cuda.synchronize()
    cold = pct([a.elapsed_time(b) for a, b in evc])
    del scrub
    log(f"[bench] per step: warm median {warm['median_ms']:.4f} ms, cold median "
        f"{cold['median_ms']:.4f} ms")

    # ---- the same step captured once in a HIP graph and replayed K times
    gstream = torch.cuda.Stream()
    gplan = hla.ForwardPlan(q, k, v, variant=variant, chunk=chunk, seg_chunks=seg, out=o,
                            workspace=ws, staged=True, stream=gstream)
    graph = torch.cuda.CUDAGraph()
    gstream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(gstream):
        gplan.run()
    torch.cuda.current_stream().wait_stream(gstream)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gstream):
        gplan.run()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(K):
        graph.replay()
    t_end.record()
    torch.cuda.synchronize()
    graph_ms = t_start.elapsed_time(t_end) / K
    log(f"[bench] graph replay: {graph_ms:.4f} ms/step")

    # the benchmarked output, kept for the CPU baseline leg's comparison
    o_host = o.float().cpu().numpy().reshape(B * H, n, dv)

    # ---- roofline of the dominant kernel (largest measured stage)
    # counter-record keys of the three stages; stage 3 at this shape runs the
    # pipelined forward kernel, whose key is stage 3's
    names = ["hla2_summary_kernel", "up_sweep_kernel", "hla2_forward_kernel"]
    shown = ["hla2_summary_kernel", "up_sweep_kernel", "hla2_forward_pipe_kernel"]
    esz = 2  # bf16
    per_token_bytes = (2 * d + 2 * dv) * esz          # q, k, v in, o out
    sumf = d * d + 2 * d * dv + 2 * d
    if dom == 2:
        alg_bytes = tokens * per_token_bytes
    elif dom == 0:
        tok_sum = B * H * min(n, (nseg - 1) * chunk * seg)
        alg_bytes = tok_sum * (2 * d + dv) * esz + B * H * (nseg - 1) * sumf * 4
    else:   # each up-sweep combine reads two summaries and writes one
        ncomb = sum(max(0, (nseg - 1) >> b) for b in range(1, 32))
        alg_bytes = B * H * ncomb * 3 * sumf * 4
    achieved = alg_bytes / (kern_ms[dom] * 1e-3) / 1e9
    traffic = stored_traffic(names[dom])
    fl_tok = flops_per_token(chunk, d, dv)
    mfma_tflops_fwd = tokens * fl_tok / (kern_ms[2] * 1e-3) / 1e12
    mfma_tflops_step = tokens * fl_tok / (ms_per_step * 1e-3) / 1e12
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": shown[dom],
                "kernel_ms": round(kern_ms[dom], 5), "alg_bytes_per_launch": int(alg_bytes),
                "cold": {"kernel_ms_median": round(kern_cold_ms, 5),
                         "achieved": round(alg_bytes / (kern_cold_ms * 1e-3) / 1e9, 2),
                         "frac": round(alg_bytes / (kern_cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}

    # ---- decode step (one token per head, AHLA state of 32 heads, d = 64)
    decode = None
    if args.decode_steps > 0:
        dw = I.WORKLOADS["ahla_n65536"]
        BHd = dw.B * dw.H
        stf = hla.state_floats("ahla", dw.d, dw.dv)
        state = torch.zeros(BHd * stf, dtype=torch.float32, device=dev)
        qd = torch.randn((dw.B, dw.H, dw.d), device=dev).to(torch.bfloat16)
        kd = torch.randn((dw.B, dw.H, dw.d), device=dev).to(torch.bfloat16)
        vd = torch.randn((dw.B, dw.H, dw.dv), device=dev).to(torch.bfloat16)
        od = torch.empty((dw.B, dw.H, dw.dv), dtype=torch.bfloat16, device=dev)
        splan = hla.StepPlan(qd, kd, vd, state, variant="ahla", out=od)
        for _ in range(10):
            splan.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.decode_steps):
            splan.run()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
        # the same steps captured in a HIP graph (64 steps per replay)
        per_graph = 64
        gsp = hla.StepPlan(qd, kd, vd, state, variant="ahla", out=od, stream=gstream)
        dgraph = torch.cuda.CUDAGraph()
        gstream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gstream):
            gsp.run()
        torch.cuda.current_stream().wait_stream(gstream)
        torch.cuda.synchronize()
        with torch.cuda.graph(dgraph, stream=gstream):
            for _ in range(per_graph):
                gsp.run()
        dgraph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.decode_steps // per_graph)
        e0.record()
        for _ in range(reps):
            dgraph.replay()
        e1.record()
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
        st_bytes = 2 * BHd * stf * 4 + BHd * (2 * dw.d + 2 * dw.dv) * 2
        decode = {"workload": "AHLA decode step, B=1 H=32 d=dv=64 bf16, fp32 state",
                  "traffic": stored_traffic("ahla_step_sliced_kernel"),
                  "us_per_step": round(us, 3), "tokens_per_s": round(BHd / (us * 1e-6), 1),
                  "us_per_step_graph": round(us_graph, 3),
                  "state_bytes_per_step": st_bytes,
                  "achieved_GBs": round(st_bytes / (us * 1e-6) / 1e9, 2),
                  "achieved_GBs_graph": round(st_bytes / (us_graph * 1e-6) / 1e9, 2)}
        log(f"[bench] decode: {us:.2f} us/step, {us_graph:.2f} us/step under graph replay")

    # ---- backward pass (HLA-2 gradients dq, dk, dv) at the benchmark shape:
    # unnormalised HLA-2 (the variant the backward supports), q, k L2-normalised
    # Gaussian rows, v and the upstream gradient ~ N(0, 1), bf16
    backward = backward_ratio = backward_decay = third_order = unmasked = None
    if args.backward_steps > 0:
        bseg = args.backward_seg_chunks or hla.backward_default_seg_chunks(B, H, n)
        bnseg = -(-n // (64 * bseg))

        def time_backward(variant, qb, kb, vb, dob, gamma=None, dgamma=None):
            bplan = hla.BackwardPlan(qb, kb, vb, dob, variant=variant, gamma=gamma,
                                     seg_chunks=bseg, dgamma=dgamma)
            for _ in range(10):
                bplan.run()
            torch.cuda.synchronize()
            t_start.record()
            for _ in range(args.backward_steps):
                bplan.run()
            t_end.record()
            torch.cuda.synchronize()
            return t_start.elapsed_time(t_end) / args.backward_steps

        # lean HBM floor: q, k, v, do read once and dq, dk, dv written once
        b_bytes = tokens * 7 * d * 2
        xb = I.make_inputs(B, H, n, d, dv, dtype="bf16", dist="l2norm", seed=w.seed + 500)
        gb = I.make_upstream_grad(B * H, n, dv, "bf16", seed=w.seed + 501)
        qb, kb, vb = (to_dev(xb[key], (B, H, n, d)) for key in ("q", "k", "v"))
        dob = to_dev(gb, (B, H, n, dv))
        del xb, gb
        bms = time_backward("hla2", qb, kb, vb, dob)
        backward = {"steps": args.backward_steps,
                    "launches_per_step": 5 + 4 * (bnseg > 1),
                    "workload": f"HLA-2 backward (dq, dk, dv), B={B} H={H} n={n} d=dv={d} bf16, "
                                "q,k L2-normalised Gaussian, v and do ~ N(0,1)",
                    "passes": "5 chunked linear-attention passes (chunk 64), each a main launch "
                              "after a segment-state launch (the last pass reuses the first's "
                              "states); dZ and dV share one pass, dK's two slots another",
                    "seg_chunks": bseg,
                    "ms_per_step": round(bms, 5), "tokens_per_s": round(tokens / (bms * 1e-3), 1),
                    "lean_bytes_per_step": b_bytes,
                    "lean_hbm_frac": round(b_bytes / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] backward: {bms:.4f} ms/step, {tokens / (bms * 1e-3) / 1e9:.3f} G tokens/s")
        # a training step's pair: the forward that keeps its keyed queries
        # z_t = S_t q_t (hla_forward_z) and the backward that takes them
        # (hla_backward_z, four passes), against hla_forward + hla_backward
        def time_plan(run):
            for _ in range(10):
                run()
            torch.cuda.synchronize()
            t_start.record()
            for _ in range(args.backward_steps):
                run()
            t_end.record()
            torch.cuda.synchronize()
            return t_start.elapsed_time(t_end) / args.backward_steps

        fplain = hla.ForwardPlan(qb, kb, vb, variant="hla2", chunk=chunk, seg_chunks=seg)
        fz = hla.ForwardPlan(qb, kb, vb, variant="hla2", chunk=chunk, seg_chunks=seg, z=True)
        fms, fzms = time_plan(fplain.run), time_plan(fz.run)
        bzplan = hla.BackwardPlan(qb, kb, vb, dob, variant="hla2", seg_chunks=bseg, z=fz.z)
        bzms = time_plan(bzplan.run)
        backward["with_forward_z"] = {
            "forward_ms": round(fms, 5), "forward_z_ms": round(fzms, 5),
            "backward_z_ms": round(bzms, 5),
            "forward_plus_backward_ms": round(fms + bms, 5),
            "forward_z_plus_backward_z_ms": round(fzms + bzms, 5)}
        log(f"[bench] forward + backward {fms + bms:.4f} ms; keeping z: forward {fzms:.4f} + "
            f"backward {bzms:.4f} = {fzms + bzms:.4f} ms")
        del fplain, fz, bzplan
        # third-order forward (variant hla3) on the same inputs: the LA pass
        # into the workspace, then the three second-order stages
        t3plan = hla.ForwardPlan(qb, kb, vb, variant="hla3", chunk=chunk, seg_chunks=seg)
        for _ in range(10):
            t3plan.run()
        torch.cuda.synchronize()
        t_start.record()
        for _ in range(args.backward_steps):
            t3plan.run()
        t_end.record()
        torch.cuda.synchronize()
        t3ms = t_start.elapsed_time(t_end) / args.backward_steps
        third_order = {"workload": f"third-order HLA forward, B={B} H={H} n={n} d=dv={d} bf16, "
                                   "q,k L2-normalised Gaussian, v ~ N(0,1)",
                       "ms_per_step": round(t3ms, 5),
                       "tokens_per_s": round(tokens / (t3ms * 1e-3), 1)}
        log(f"[bench] third-order forward: {t3ms:.4f} ms/step")
        del qb, kb, vb, t3plan
        # the benchmark's own variant and inputs: ratio HLA-2 on q, k, v above
        rms = time_backward("hla2_ratio", q, k, v, dob)
        backward_ratio = {"steps": args.backward_steps,
                          "workload": f"ratio HLA-2 backward, the forward's inputs (B={B} H={H} "
                                      f"n={n} d=dv={d} bf16), do ~ N(0,1)",
                          "passes": "8 chunked linear-attention passes and a row-wise kernel: "
                                    "num and den recomputed, then the HLA-2 passes with "
                                    "upstream do/den and one pass for den's term",
                          "seg_chunks": bseg,
                          "ms_per_step": round(rms, 5),
                          "tokens_per_s": round(tokens / (rms * 1e-3), 1),
                          "lean_hbm_frac": round(b_bytes / (rms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] ratio backward: {rms:.4f} ms/step, {tokens / (rms * 1e-3) / 1e9:.3f} G tokens/s")
        # HLA-2 with per-head decays on the same inputs, without and with the
        # decay gradient (two more launches over q, k, Z, dq, dk, dZ)
        gam = np.random.default_rng(w.seed + 502).uniform(0.95, 0.999, H).astype(np.float32)
        dms = time_backward("hla2", q, k, v, dob, gamma=gam)
        dgms = time_backward("hla2", q, k, v, dob, gamma=gam, dgamma=True)
        backward_decay = {"steps": args.backward_steps,
                          "workload": f"HLA-2 backward with decays g_h ~ U[0.95, 0.999], the "
                                      f"forward's inputs (B={B} H={H} n={n} d=dv={d} bf16), "
                                      "do ~ N(0,1)",
                          "ms_per_step": round(dms, 5),
                          "ms_per_step_with_dgamma": round(dgms, 5),
                          "dgamma_passes": "fp32 (widened copies of the bf16 inputs)",
                          "dgamma_bytes": tokens * 6 * d * 4}
        log(f"[bench] decay backward: {dms:.4f} ms/step, with dL/dgamma {dgms:.4f} ms/step")
        # unmasked (non-causal) operators on the forward's inputs
        unmasked = {}
        for uv in ("hla2", "ahla"):
            uo = torch.empty_like(q)
            uws = torch.empty(max(hla.unmasked_workspace_bytes(B, H, n, d), 1), dtype=torch.uint8,
                              device=dev)
            for _ in range(10):
                hla.hla_unmasked_forward(q, k, v, uv, out=uo, workspace=uws)
            torch.cuda.synchronize()
            t_start.record()
            for _ in range(args.backward_steps):
                hla.hla_unmasked_forward(q, k, v, uv, out=uo, workspace=uws)
            t_end.record()
            torch.cuda.synchronize()
            ums = t_start.elapsed_time(t_end) / args.backward_steps
            unmasked[uv] = {"ms_per_step": round(ums, 5), "tokens_per_s": round(tokens / (ums * 1e-3), 1)}
            log(f"[bench] unmasked {uv}: {ums:.4f} ms/step")
            del uo, uws
        del dob

    # ---- CPU baseline: the oracle on the same inputs, all heads; its output
    # is also compared with the benchmarked GPU output, every element
    cpu = None
    rel = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.max_threads()
        reps = 0
        t0 = time.perf_counter()
        while True:
            want = oracle.hla2(x["q"], x["k"], x["v"], ratio=True, threads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= args.cpu_seconds or reps >= 1000:
                break
        cpu = {"value": round(reps * tokens / dt, 1), "unit": "tokens/s", "cores": threads,
               "kind": "oracle", "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
               "sample": f"the whole workload ({B * H} heads x {n} tokens) {reps} times over, "
                         f"fp64 serial recurrence, one head per thread, {dt:.2f} s wall"}
        log(f"[bench] cpu oracle: {reps} passes in {dt:.2f} s on {threads} threads")
        rel = float(np.linalg.norm(o_host - want) / np.linalg.norm(want))
        log(f"[bench] GPU output vs oracle (all {B * H} heads): rel_l2 {rel:.3e}")
        del want

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "variant": variant, "B": B, "H": H, "n": n, "d": d,
                   "dv": dv, "chunk": chunk, "seg_chunks": seg, "segments": nseg,
                   "global_batch": B, "seq_len": n, "parallelism": "single-gpu"},
        "roofline": roofline,
        "mfma": {"alg_flops_per_token": fl_tok, "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                 "forward_kernel_tflops": round(mfma_tflops_fwd, 2),
                 "forward_kernel_frac": round(mfma_tflops_fwd / BF16_MFMA_PEAK_TFLOPS, 4),
                 "whole_step_tflops": round(mfma_tflops_step, 2),
                 "whole_step_frac": round(mfma_tflops_step / BF16_MFMA_PEAK_TFLOPS, 4)},
        "stages_ms": {"summary": round(stage_ms[0], 5), "up_sweep": round(stage_ms[1], 5),
                      "prefix_and_forward": round(stage_ms[2], 5)},
        "kernel_ms": {"summary": round(kern_ms[0], 5), "up_sweep": round(kern_ms[1], 5),
                      "prefix_and_forward": round(kern_ms[2], 5)},
        "per_step_warm": warm,
        "per_step_cold": cold,
        "graph_ms_per_step": round(graph_ms, 5),
        "parity_rel_l2": rel,
        "decode": decode,
        "backward": backward,
        "backward_ratio": backward_ratio,
        "backward_decay": backward_decay,
        "unmasked": unmasked,
        "third_order": third_order,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo (Linux)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
