"""Benchmark of the LoRA hot path on one MI355X.

One step = one single-adapter forward + backward pass over a batch:
lora_fwd (Y += s*(X*A)*B), lora_bwd_dx_da (dX, dA), lora_bwd_db (dB), by
default on the largest bf16-in / fp32-out workload, the MLP-up shape M = 16384
tokens, K = 4096, L = 14336, rank 64, s = 0.5 (synthetic seeded data, see
synth/); --workload selects the 8192 x 4096 x 4096, rank 16 one instead.
Inputs are resident in HBM before
the timed region; several copies of the streamed tensors rotate so that
successive steps do not read the previous step's data from the 256 MB
Infinity Cache.

Prints ONE JSON line with the throughput (tokens/s over the whole step), the
step's algorithmic HBM bandwidth, a roofline entry for the dominant kernel
(the fused forward: algorithmic bytes / its average launch duration, from
HIP events that the kernel's own dispatch stamps on its stream during the
timed steps; see lora_timing_* in include/lora.h), and the CPU oracle's
throughput on the same workload as a baseline.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       python bench.py ... --copy-probe      (adds 1 GiB plain copies after the
                                             timed region, the calibration for
                                             the byte counters)
       python bench.py --traffic-summary FETCH_CSV WRITE_CSV [--workload NAME]
           reads two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE,
           then WRITE_SIZE) of a bench run with --copy-probe and writes the
           roofline kernel's HBM bytes per launch to profiles/.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "LoRA fwd+bwd tokens/s and achieved HBM GB/s (% of roofline), 1×MI355X"

WORKLOADS = {
    # name: (M, K, L, r, scale, seed)
    "single-bf16-M8192-K4096-L4096-r16": (8192, 4096, 4096, 16, 2.0, 2),
    "single-bf16-M16384-K4096-L14336-r64": (16384, 4096, 14336, 64, 0.5, 3),
}
DEFAULT_WORKLOAD = "single-bf16-M16384-K4096-L14336-r64"

# The kernels the roofline entry is about, per workload: what lora_fwd
# launches at that shape (weights used in place, so no packing launch): the
# fused shrink+expand kernel for the 134 MB output; for the 940 MB output the
# split schedule's shrink kernel and column-band expand (both are the
# forward's dominant work, timed together).
ROOFLINE_KERNEL = {
    "single-bf16-M8192-K4096-L4096-r16": ["fused_kernel"],
    "single-bf16-M16384-K4096-L14336-r64": ["shrink_kernel", "expand_band_kernel"],
}
# How those launches are told apart from the same templates' backward
# instances in a profile (the last template argument of each is WT, the
# backward's transposed-weight flag, false in the forward): the forward ones
# accumulate into Y (lora::OutAdd with EMIT_G = false in fused_kernel;
# lora::OutAdd in expand_band_kernel, the backward's band expands running
# inside band_tn_kernel) or write only fragments (EMIT_G = false,
# EMIT_F = true in shrink_kernel).
ROOFLINE_PATTERN = {
    "fused_kernel": r"\bfused_kernel<.*, lora::OutAdd, false, false>",
    "shrink_kernel": r"\bshrink_kernel<.*, false, true, false>",
    "expand_band_kernel": r"\bexpand_band_kernel<.*, lora::OutAdd, false>",
}


def roofline_grid(kernel, workload):
    """Work-items of the forward's launch of `kernel` (None: any): the band
    expand runs 256 threads per (256-column band, group of four 32-token
    tiles)."""
    if kernel != "expand_band_kernel":
        return None
    M, _K, Lc, _r, _s, _seed = WORKLOADS[workload]
    return -(-Lc // 256) * -(-(-(-M // 32)) // 4) * 256
COPY_PROBE_BYTES = 1 << 30
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def algorithmic_bytes(M, K, L, r, es=2):
    """Bytes each call must move at least once (streamed tensors once, weights
    once, fp32 outputs; on-chip intermediates not counted)."""
    fwd = M * (es * K + 8 * L) + es * r * (K + L)
    dxda = M * (es * L + 4 * K + es * K) + es * r * (K + L) + 4 * K * r
    db = M * (es * K + es * L) + es * r * K + 4 * r * L
    return {"fwd": fwd, "dx_da": dxda, "db": db, "dx_da_accumulate": dxda + 4 * M * K}


def source_digest(paths):
    """Digest of the kernel sources with comments and blank space removed, so
    that a comment-only edit keeps counter records valid."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


KERNEL_SOURCES = ["lora_rank_adapter_amd/csrc/lora_single.hip", "lora_rank_adapter_amd/csrc/lora_device.hpp"]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{'+'.join(ROOFLINE_KERNEL[workload])}_{workload}.json")


def traffic_from_profile(workload):
    """HBM traffic of the roofline kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest(KERNEL_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_per_dispatch(path, counter, pattern, grid=None):
    """{dispatch id: counter value} (KiB for the byte counters) over the
    dispatches whose kernel name matches the regex `pattern` (and whose grid
    has `grid` work-items, if given)."""
    per = {}
    rx = re.compile(pattern)
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if grid is not None and int(row["Grid_Size"]) != grid:
                continue
            if row["Counter_Name"] == counter and rx.search(row["Kernel_Name"]):
                d = int(row["Dispatch_Id"])
                per[d] = per.get(d, 0.0) + float(row["Counter_Value"])
    return per


def _kernel_mean(path, counter, pattern, grid=None):
    per = _counter_per_dispatch(path, counter, pattern, grid)
    if not per:
        raise SystemExit(f"no dispatch of {pattern!r} with {counter} in {path}")
    return statistics.mean(per.values()), len(per)


def copy_probe(dev):
    """Three plain copies of COPY_PROBE_BYTES (the byte counters' calibration)."""
    import torch
    src_t = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    dst_t = torch.empty_like(src_t)
    for _ in range(3):
        dst_t.copy_(src_t)
    torch.cuda.synchronize()
    del src_t, dst_t


def _copy_probe_kib(path, counter):
    """The counter for the 1 GiB copies of --copy-probe: the last three copy
    dispatches of the run (the input clones before them are smaller)."""
    per = _counter_per_dispatch(path, counter, COPY_KERNEL)
    last = [per[d] for d in sorted(per)[-3:]]
    if len(last) < 3:
        raise SystemExit(f"{path}: fewer than 3 copy dispatches; was the run made with --copy-probe?")
    return statistics.mean(last)


def traffic_summary(fetch_csv, write_csv, workload, command):
    """HBM bytes per lora_fwd call of the roofline kernel(s): FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by bytes-moved / counter-reading
    of the plain 1 GiB copy that ran in the same process."""
    kern = ROOFLINE_KERNEL[workload]
    f_copy = _copy_probe_kib(fetch_csv, "FETCH_SIZE") * 1024
    w_copy = _copy_probe_kib(write_csv, "WRITE_SIZE") * 1024
    f_scale, w_scale = COPY_PROBE_BYTES / f_copy, COPY_PROBE_BYTES / w_copy
    fetch = [_kernel_mean(fetch_csv, "FETCH_SIZE", ROOFLINE_PATTERN[k], roofline_grid(k, workload)) for k in kern]
    write = [_kernel_mean(write_csv, "WRITE_SIZE", ROOFLINE_PATTERN[k], roofline_grid(k, workload)) for k in kern]
    f_k = sum(v for v, _ in fetch)
    w_k = sum(v for v, _ in write)
    n_f = [n for _, n in fetch]
    n_w = [n for _, n in write]
    M, K, Lc, r, _, _ = WORKLOADS[workload]
    rec = {
        "kernels": kern,
        "workload": workload,
        "command": command,
        "source_digest": source_digest(KERNEL_SOURCES),
        "copy_probe_bytes": COPY_PROBE_BYTES,
        "copy_fetch_kib": f_copy / 1024, "copy_write_kib": w_copy / 1024,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "kernel_fetch_kib": f_k, "kernel_write_kib": w_k, "dispatches": [n_f, n_w],
        "hbm_bytes_per_launch": f_k * 1024 * f_scale + w_k * 1024 * w_scale,
        "algorithmic_bytes_per_launch": algorithmic_bytes(M, K, Lc, r)["fwd"],
    }
    rec["traffic_over_algorithmic"] = rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
    with open(traffic_path(workload), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def multi_traffic_summary(fetch_csv, write_csv, command):
    """HBM bytes per dispatch of the multi-adapter kernels (a --multi-only run
    with --copy-probe): FETCH_SIZE and WRITE_SIZE scaled like the forward's,
    per (kernel, grid size); the prefill shrink and expand (the row-split
    shrink, the band expand's largest grid) against their algorithmic bytes."""
    import numpy as np

    import synth
    f_scale = COPY_PROBE_BYTES / (_copy_probe_kib(fetch_csv, "FETCH_SIZE") * 1024)
    w_scale = COPY_PROBE_BYTES / (_copy_probe_kib(write_csv, "WRITE_SIZE") * 1024)

    def per_kernel(path, counter):
        out = {}
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter or "lora::" not in row["Kernel_Name"]:
                    continue
                name = re.sub(r"^void ", "", row["Kernel_Name"]).split("(")[0]
                key = (name, int(row["Grid_Size"]), int(row["Dispatch_Id"]))
                out[key] = out.get(key, 0.0) + float(row["Counter_Value"])
        agg = {}
        for (name, grid, _), v in out.items():
            agg.setdefault((name, grid), []).append(v)
        return agg

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    # algorithmic bytes of the prefill calls, as multi_lora_figures counts them
    ts, rk, _, _ = synth.config5_routing()
    K, slices, r_max = 8192, (8192, 1024, 1024), 128
    S, n, SO = rk.shape[0], len(slices), sum(slices)
    rho = np.clip(rk, 0, r_max)
    act = (ts >= 0) & (ts < S) & (rho[np.clip(ts, 0, S - 1)] > 0)
    live = int(rho[np.unique(ts[act])].sum())
    na, rho_sum = int(act.sum()), int(rho[ts[act]].sum())
    sh_bytes = na * 2 * K + 2 * K * n * live + 4 * n * rho_sum
    ex_bytes = 4 * n * rho_sum + 2 * SO * live + 8 * SO * na
    lines = ["# Multi-adapter kernels: HBM bytes per dispatch (rocprofv3 byte counters)", "",
             "Commands (from the repository root; one counter per run):", "", "```", command, "```", "",
             f"FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f}: the bytes a plain 1 GiB copy "
             "moves per counter unit in the same run (`--copy-probe`). The run covers the decode workloads (256 and "
             "1024 tokens) and the prefill workload (16731 tokens); kernels are told apart by grid size.", "",
             "| kernel | grid | dispatches | MB fetched | MB written |", "|---|---|---|---|---|"]
    rows = []
    for key in sorted(set(fetch) | set(write)):
        fv, wv = fetch.get(key, [0.0]), write.get(key, [0.0])
        fmb = statistics.mean(fv) * 1024 * f_scale / 1e6
        wmb = statistics.mean(wv) * 1024 * w_scale / 1e6
        rows.append((key, len(fv), fmb, wmb))
        lines.append(f"| `{key[0]}` | {key[1]} | {len(fv)} | {fmb:.1f} | {wmb:.1f} |")

    def largest(name):
        cand = [r for r in rows if re.search(name, r[0][0])]
        return max(cand, key=lambda r: r[0][1]) if cand else None
    lines += ["", "Prefill (46 slots, r_max 128):"]
    for label, pat, alg in (("shrink (row-split)", r"slot_shrink_rows_kernel", sh_bytes),
                            ("expand_fused (column band)", r"slot_expand_band_kernel", ex_bytes)):
        r = largest(pat)
        if r:
            tot = (r[2] + r[3]) * 1e6
            lines.append(f"- {label}: {r[2]:.1f} MB fetched + {r[3]:.1f} MB written = {tot / 1e6:.1f} MB against "
                         f"{alg / 1e6:.1f} MB algorithmic ({tot / alg:.3f}x)")
    path = os.path.join(ROOT, "profiles", "traffic_multi-adapter_decode-T256-T1024_prefill-T16731.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Hardware counters the --counter-summary tables use (one rocprofv3 --pmc pass:
# 7 SQ counters and GRBM_GUI_ACTIVE, within one pass's limits).
PMC_COUNTERS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"]
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def counter_summary(csv_path, name, command):
    """Per kernel (mean over its dispatches), with the kernel's busy cycles
    G = GRBM_GUI_ACTIVE / 8 (the counter collection sums the GUI-active
    cycles of the 8 XCDs, each with its own GRBM): MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (G * SIMDs); mean resident waves per CU =
    4 * SQ_WAVE_CYCLES / (G * CUs) (SQ_WAVE_CYCLES counts in units of 4
    cycles); bf16 MFMA TFLOP/s = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16 / (G at
    2.4 GHz); LDS bank-conflict cycles per LDS instruction cycle =
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE."""
    per = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            key = (row["Kernel_Name"], int(row["Dispatch_Id"]))
            d = per.setdefault(key, {})
            d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    kernels = {}
    for (kname, _), d in per.items():
        kernels.setdefault(kname, []).append(d)
    lines = [f"# Hardware counters: {name}", "", "Command (from the repository root; outputs under gpurun_out/):", "",
             "```", command, "```", "",
             "Counters: " + ", ".join(PMC_COUNTERS) + ". Per kernel, means over its dispatches:",
             "G = GRBM_GUI_ACTIVE / 8 (the collection sums the 8 XCDs' GUI-active cycles; G / 2.4 GHz "
             "matches the kernel-trace duration); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (G x 1024 SIMDs); "
             "waves/CU = 4 x SQ_WAVE_CYCLES / (G x 256 CUs); bf16 MFMA TFLOP/s = 512 x "
             "SQ_INSTS_VALU_MFMA_MOPS_BF16 / (G / 2.4 GHz); LDS conflict = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
             "| kernel | dispatches | µs (G / 2.4 GHz) | MFMA busy | waves/CU | bf16 MFMA TFLOP/s | LDS conflict |",
             "|---|---|---|---|---|---|---|"]
    rows = []
    for kname, ds in kernels.items():
        if not kname.startswith("void lora::") and not kname.startswith("lora::"):
            continue

        def mean(c):
            return statistics.mean(d.get(c, 0.0) for d in ds)
        gui = mean("GRBM_GUI_ACTIVE") / XCD_NUM
        if gui <= 0:
            continue
        us = gui / 2.4e3
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (gui * SIMD_NUM)
        waves = 4.0 * mean("SQ_WAVE_CYCLES") / (gui * CU_NUM)
        tflops = 512.0 * mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") / (us * 1e-6) / 1e12
        lds = mean("SQ_LDS_IDX_ACTIVE")
        conf = mean("SQ_LDS_BANK_CONFLICT") / lds if lds > 0 else 0.0
        short = re.sub(r"^void ", "", kname).replace("(lora::FusedArgs)", "").replace("(lora::TnArgs)", "")
        short = re.sub(r"\(.*\)$", "", short)
        rows.append((us, f"| `{short[:90]}` | {len(ds)} | {us:.1f} | {busy:.3f} | {waves:.2f} | {tflops:.1f} | "
                         f"{conf:.3f} |"))
    lines += [r for _, r in sorted(rows, reverse=True)]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", f"counters_{name}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_summary(csv_path, name, command):
    """Kernel statistics of a rocprofv3 --kernel-trace --stats run as a table."""
    with open(csv_path, newline="") as f:
        rows = list(csv.DictReader(f))
    lines = [f"# rocprofv3 kernel statistics: {name}", "", "Command (from the repository root; outputs under "
             "gpurun_out/):", "", "```", command, "```", "",
             "| kernel | calls | avg µs | min µs | max µs | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        kname = re.sub(r"^void ", "", r["Name"])
        kname = re.sub(r"\((lora::)?\w+Args\)$", "", kname)
        lines.append(f"| `{kname[:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    # rocprofv3's statistics merge a kernel's launches of every shape; the
    # trace beside them gives the mean per grid size (one kernel serves
    # several calls, e.g. the column-band expand of the forward and of dX)
    trace = os.path.join(os.path.dirname(csv_path), "run_kernel_trace.csv")
    if os.path.exists(trace):
        per = {}
        with open(trace, newline="") as f:
            for r in csv.DictReader(f):
                if "lora::" not in r["Kernel_Name"]:
                    continue
                kname = re.sub(r"^void ", "", r["Kernel_Name"])
                kname = re.sub(r"\((lora::)?\w+Args\)$", "", kname)
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                per.setdefault((kname, grid), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", "Per launch shape (kernel trace in the same directory):", "",
                  "| kernel | grid (threads) | launches | avg µs | median µs |", "|---|---|---|---|---|"]
        for (kname, grid), ds in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| `{kname[:100]}` | {grid} | {len(ds)} | {statistics.mean(ds):.2f} | "
                         f"{statistics.median(ds):.2f} |")
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{name}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(case, budget_s=8.0):
    """The float64 CPU oracle (numpy, as it stands) on a bounded sample of the
    batch: the first `tokens` rows of X, dY and Y0 with the full weights, one
    forward + lora_bwd_dx_da + lora_bwd_db per run, median over repeated runs
    for about `budget_s` seconds; on every thread the host's BLAS uses, then on
    one. Tokens/s scale linearly with the sample (every op is per-token work
    plus the token sums of dA and dB)."""
    import threadpoolctl

    import oracle

    def measure(tokens):
        X, dY, Y0 = case.X[:tokens], case.dY[:tokens], case.Y0[:tokens]
        times = []
        t_start = time.perf_counter()
        while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 200):
            t0 = time.perf_counter()
            oracle.lora_fwd(X, case.A, case.B, Y0, case.scale)
            oracle.lora_bwd_dx_da(X.T, dY, case.B.T, case.A.T, case.scale)
            oracle.lora_bwd_db(case.A.T, X.T, dY, case.scale)
            times.append(time.perf_counter() - t0)
        return tokens / statistics.median(times), len(times), sum(times)

    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    n_all = min(case.M, 2048)
    v_all, runs_all, t_all = measure(n_all)
    n_one = min(case.M, 256)
    with threadpoolctl.threadpool_limits(1):
        v_one, runs_one, t_one = measure(n_one)
    return {
        "value": v_all,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {n_all} of {case.M} tokens (full weights), fwd + bwd_dx_da + bwd_db in float64 "
                  f"numpy, median of {runs_all} runs ({t_all:.1f} s)",
        "one_core": {"value": v_one, "unit": "tokens/s", "cores": 1,
                     "sample": f"first {n_one} tokens, median of {runs_one} runs ({t_one:.1f} s)"},
        "host": {"nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(), "cpu_model": _cpu_model()},
    }


def multi_lora_figures(dev, reps=20, graph=True):
    """Kernel times of the slot-addressed ops on the decode and prefill
    workloads (routing from synth's seeded laws; values drawn on the device
    with the same laws), with their algorithmic bytes: activations once per
    active token, each used slot's live adapter rows once, h once, y read and
    written for active tokens. Whole input sets (x, adapters, y, h) rotate, at
    least 1 GB of them, so that no repetition finds the previous one's data in
    the 256 MB Infinity Cache."""
    import numpy as np
    import torch

    import lora_rank_adapter_amd as L
    import synth

    gen = torch.Generator(device=dev)
    gen.manual_seed(5)

    def timed(f, n, host=False):
        """Time per call of n calls in a row. GPU time by default: the calls
        queue behind a short GPU spin, so the GPU runs them back to back
        whatever the host's submission cost (about 13 us per Python call,
        more than a decode kernel takes); host=True times them as submitted."""
        f(0)
        torch.cuda.synchronize()
        if not host:
            torch.cuda._sleep(20_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            f(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    out = {}
    rng4 = np.random.default_rng(4)
    ts4, rk4 = synth.decode_routing(256, 32, 64, (0, 8, 16, 32, 64), 0.1, rng4)
    ts4k, rk4k = synth.decode_routing(1024, 32, 64, (0, 8, 16, 32, 64), 0.1, np.random.default_rng(41))
    ts5, rk5, _lengths, _rng5 = synth.config5_routing()
    for name, ts_np, rk_np, K, slices, r_max in (
            ("decode-T256-K4096-qkv-S32-rmax64", ts4, rk4, 4096, (4096, 1024, 1024), 64),
            ("decode-T1024-K4096-qkv-S32-rmax64", ts4k, rk4k, 4096, (4096, 1024, 1024), 64),
            ("prefill-K8192-qkv-S128-rmax128", ts5, rk5, 8192, (8192, 1024, 1024), 128)):
        T, S, n, SO = ts_np.shape[0], rk_np.shape[0], len(slices), sum(slices)
        set_bytes = 2 * T * K + 2 * S * n * r_max * K + 2 * S * SO * r_max + 4 * T * SO + 4 * T * n * r_max
        nsets = max(2, min(24, -(-(1 << 30) // set_bytes)))
        ts = torch.from_numpy(ts_np).to(dev)
        rk = torch.from_numpy(rk_np).to(dev)
        xs = [torch.randn((T, K), device=dev, generator=gen).to(torch.bfloat16) for _ in range(nsets)]
        as_ = [(torch.randn((S, n * r_max, K), device=dev, generator=gen) / K ** 0.5).to(torch.bfloat16)
               for _ in range(nsets)]
        bs = [(torch.randn((S, SO, r_max), device=dev, generator=gen) / 8).to(torch.bfloat16) for _ in range(nsets)]
        sc = torch.rand(S, device=dev, generator=gen) * 1.5 + 0.5
        ys = [torch.randn((T, SO), device=dev, generator=gen) for _ in range(nsets)]
        hs = [torch.zeros((T, n, r_max), device=dev) for _ in range(nsets)]
        addr = L.Addressing(ts, S)
        t_group = timed(lambda i: L.lora_addressing_build(addr, rk, r_max), reps)
        t_shrink = timed(lambda i: L.lora_shrink(xs[i % nsets], as_[i % nsets], addr, rk, n, r_max,
                                                 h=hs[i % nsets]), reps)
        t_expand = timed(lambda i: L.lora_expand_fused(hs[i % nsets], bs[i % nsets], addr, rk, sc, ys[i % nsets],
                                                       slices, r_max), reps)
        t_apply = timed(lambda i: L.lora_apply_linear(xs[i % nsets], ys[i % nsets], as_[i % nsets], bs[i % nsets],
                                                      addr, rk, sc, slices, r_max, h=hs[i % nsets]), reps)
        rho = np.clip(rk_np, 0, r_max)
        act = (ts_np >= 0) & (ts_np < S) & (rho[np.clip(ts_np, 0, S - 1)] > 0)
        used = np.unique(ts_np[act])
        na = int(act.sum())
        live = int(rho[used].sum())
        rho_sum = int(rho[ts_np[act]].sum())
        sh_bytes = na * 2 * K + 2 * K * n * live + 4 * n * rho_sum
        ex_bytes = 4 * n * rho_sum + 2 * SO * live + 8 * SO * na
        out[name] = {
            "tokens": T, "active_tokens": na, "used_slots": int(len(used)), "rotating_input_sets": nsets,
            "grouping_us": t_group,
            "shrink_us": t_shrink, "shrink_gbs": sh_bytes / t_shrink / 1e3,
            "expand_fused_us": t_expand, "expand_fused_gbs": ex_bytes / t_expand / 1e3,
            "expand_fused_frac": ex_bytes / t_expand / 1e3 / HBM_PEAK_GBS,
            # one call; one launch with h on chip where the library takes that
            # form (the 1024-token decode), else the shrink and the expand
            "apply_linear_us": t_apply,
            "apply_linear_gbs": (sh_bytes + ex_bytes - 8 * n * rho_sum) / t_apply / 1e3,
        }
        if T <= 4096 and graph:
            # a serving step's calls (grouping, then apply_linear) back to
            # back: as submitted eagerly, as one captured HIP graph replayed
            # per step (no host sync or data-dependent shape in them, so a
            # serving loop can capture them), and the GPU time of the eager
            # step (queued behind a spin)
            def seq(i):
                j = i % nsets
                L.lora_addressing_build(addr, rk, r_max)
                L.lora_apply_linear(xs[j], ys[j], as_[j], bs[j], addr, rk, sc, slices, r_max, h=hs[j])

            side = torch.cuda.Stream(device=dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                seq(0)
            torch.cuda.current_stream(dev).wait_stream(side)
            torch.cuda.synchronize()
            step_graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(step_graph):
                seq(0)
            out[name]["step_eager_us"] = timed(seq, reps, host=True)
            out[name]["step_graph_us"] = timed(lambda i: step_graph.replay(), reps, host=True)
            out[name]["step_gpu_us"] = timed(seq, reps)
            del step_graph
        del xs, as_, bs, ys, hs
    # gather_shrink over the 128256-row embedding adapter table (4.2 GB, rank index contiguous)
    T, S, r_max, V = ts5.shape[0], 128, 128, 128256
    tab = torch.randn((S, V, r_max), device=dev, generator=gen).to(torch.bfloat16).permute(0, 2, 1)
    ids = torch.randint(0, V, (T,), device=dev, generator=gen, dtype=torch.int32)
    ids[torch.rand(T, device=dev, generator=gen) < 0.05] = -1
    rk = torch.from_numpy(rk5).to(dev)
    addr = L.lora_addressing_build(L.Addressing(torch.from_numpy(ts5).to(dev), S), rk, r_max)
    h = torch.zeros((T, 1, r_max), device=dev)
    out["gather_shrink-V128256-S128-rmax128"] = {
        "tokens": T, "us": timed(lambda i: L.lora_gather_shrink(ids, tab, addr, rk, r_max, h=h), reps)}
    del tab
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-multi", action="store_true", help="skip the multi-adapter serving figures")
    ap.add_argument("--multi-only", action="store_true",
                    help="only the multi-adapter serving figures (no single-adapter step)")
    ap.add_argument("--multi-reps", type=int, default=20, help="repetitions per multi-adapter figure")
    ap.add_argument("--no-graph", action="store_true", help="skip the decode step's HIP-graph replays")
    ap.add_argument("--counter-summary", metavar="CSV",
                    help="summarise a rocprofv3 --pmc counter_collection.csv (MFMA busy, occupancy, LDS "
                         "bank conflicts per kernel) into profiles/")
    ap.add_argument("--summary-name", default="", help="file name stem for --counter-summary / --stats-summary")
    ap.add_argument("--stats-summary", metavar="CSV",
                    help="summarise a rocprofv3 --kernel-trace --stats kernel_stats.csv into profiles/")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--multi-traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="byte counters of a --multi-only --copy-probe run -> profiles/")
    ap.add_argument("--command", default="", help="the profiled command, recorded with --traffic-summary")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.workload, args.command)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.summary_name, args.command)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary, args.summary_name, args.command)
        return
    if args.multi_traffic_summary:
        multi_traffic_summary(*args.multi_traffic_summary, args.command)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the single-adapter and multi-adapter paths run on one MI355X and are not sharded here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lora_rank_adapter_amd as L
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    L.load_library()
    dev = torch.device("cuda:0")
    if args.multi_only:
        print(json.dumps({"multi_lora": multi_lora_figures(dev, reps=args.multi_reps, graph=not args.no_graph)}),
              flush=True)
        if args.copy_probe:
            copy_probe(dev)
        return
    M, K, Lc, r, scale, seed = WORKLOADS[args.workload]
    case = synth.single_adapter(M, K, Lc, r, seed=seed, dtype="bf16", scale=scale, name=args.workload)

    def bf16(a):
        return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)

    A_w = bf16(np.ascontiguousarray(case.A.T))   # lora_A weight, r x K
    B_w = bf16(np.ascontiguousarray(case.B.T))   # lora_B weight, L x r
    X0 = bf16(case.X)
    dY0 = bf16(case.dY)
    set_bytes = M * (2 * K + 2 * Lc + 4 * Lc + 4 * K)
    n_sets = max(2, min(6, int(np.ceil(1.0e9 / set_bytes))))
    sets = []
    for i in range(n_sets):
        sets.append({
            "X": X0.clone(), "dY": dY0.clone(),
            "Y": torch.zeros((M, Lc), dtype=torch.float32, device=dev),
            "dX": torch.empty((M, K), dtype=torch.float32, device=dev),
        })
    del X0, dY0
    dA = torch.empty((K, r), dtype=torch.float32, device=dev)
    dB = torch.empty((r, Lc), dtype=torch.float32, device=dev)
    ws0 = torch.empty(max(1, L.lora_workspace_bytes(L.LORA_OP_FWD, M, K, Lc, r, torch.bfloat16)), dtype=torch.uint8,
                      device=dev)
    ws1 = torch.empty(L.lora_workspace_bytes(L.LORA_OP_BWD_DX_DA, M, K, Lc, r, torch.bfloat16), dtype=torch.uint8,
                      device=dev)
    ws2 = torch.empty(L.lora_workspace_bytes(L.LORA_OP_BWD_DB, M, K, Lc, r, torch.bfloat16), dtype=torch.uint8,
                      device=dev)

    def step(i, ev=None, time_fwd_kernel=False):
        s = sets[i % n_sets]
        if ev is not None:
            ev[0].record()
        if time_fwd_kernel:
            L.lora_timing_resume()
        L.lora_fwd(s["X"], A_w.t(), B_w.t(), s["Y"], scale, workspace=ws0)
        if time_fwd_kernel:
            L.lora_timing_pause()
        if ev is not None:
            ev[1].record()
        L.lora_bwd_dx_da(s["X"].t(), s["dY"], B_w, A_w, scale, dx=s["dX"], dA=dA, workspace=ws1)
        if ev is not None:
            ev[2].record()
        L.lora_bwd_db(A_w, s["X"].t(), s["dY"], scale, dB=dB, workspace=ws2)
        if ev is not None:
            ev[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: whole steps between two events on torch's current stream
    # (the stream the library launches on). The forward's kernels are launched
    # with the library's kernel timing on: HIP events that their dispatch
    # stamps at kernel start and end (the roofline kernel's launch duration).
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # events for the timed forward launches exist before the timed region
    L.lora_timing_reserve(4 * args.steps)
    L.lora_timing_begin()
    L.lora_timing_pause()
    t_begin.record()
    for i in range(args.steps):
        step(args.warmup + i, time_fwd_kernel=True)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_begin.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    fwd_kernel_total_ms, fwd_launches = L.lora_timing_read()
    fwd_kernel_ms = fwd_kernel_total_ms / args.steps      # kernel time per lora_fwd call
    # per-call split (events around each call, informative), from a separate pass
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(10)]
    for i in range(10):
        step(i, evb[i])
    torch.cuda.synchronize()
    fwd_ms = statistics.median(e[0].elapsed_time(e[1]) for e in evb)
    dxda_ms = statistics.median(e[1].elapsed_time(e[2]) for e in evb)
    db_ms = statistics.median(e[2].elapsed_time(e[3]) for e in evb)
    # the accumulating variant of lora_bwd_dx_da (dX added to the base layer's
    # gradient), outside the step: events around each call on the same sets
    eva = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
    for i in range(10):
        s_ = sets[i % n_sets]
        eva[i][0].record()
        L.lora_bwd_dx_da_accumulate(s_["X"].t(), s_["dY"], B_w, A_w, scale, s_["dX"], dA=dA, workspace=ws1)
        eva[i][1].record()
    torch.cuda.synchronize()
    dxda_acc_ms = statistics.median(e[0].elapsed_time(e[1]) for e in eva)

    if args.copy_probe:
        copy_probe(dev)

    ab = algorithmic_bytes(M, K, Lc, r)
    step_bytes = ab["fwd"] + ab["dx_da"] + ab["db"]
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    fwd_gbs = ab["fwd"] / (fwd_ms * 1e-3) / 1e9
    fwd_kernel_gbs = ab["fwd"] / (fwd_kernel_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(args.workload)

    out = {
        "metric": METRIC,
        "value": M / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": M, "in_features": K, "out_features": Lc, "rank": r,
                   "scale": scale, "outputs": "fp32", "rotating_input_sets": n_sets},
        "hbm_gbs": step_gbs,
        "hbm_frac": step_gbs / HBM_PEAK_GBS,
        "per_call_ms": {"lora_fwd": fwd_ms, "lora_bwd_dx_da": dxda_ms, "lora_bwd_db": db_ms,
                        "lora_bwd_dx_da_accumulate": dxda_acc_ms},
        "per_call_algorithmic_gbs": {
            "lora_fwd": fwd_gbs,
            "lora_bwd_dx_da": ab["dx_da"] / (dxda_ms * 1e-3) / 1e9,
            "lora_bwd_db": ab["db"] / (db_ms * 1e-3) / 1e9,
            "lora_bwd_dx_da_accumulate": ab["dx_da_accumulate"] / (dxda_acc_ms * 1e-3) / 1e9,
        },
        "roofline": {
            "kernel": " + ".join(ROOFLINE_KERNEL[args.workload]) + " (lora_fwd)",
            "bound": "hbm",
            "achieved": fwd_kernel_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": fwd_kernel_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel_us": fwd_kernel_ms * 1e3,
            "launches_per_call": fwd_launches / args.steps,
            "algorithmic_bytes": ab["fwd"],
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(case),
    }
    if not args.no_multi:
        del sets
        torch.cuda.empty_cache()
        out["multi_lora"] = multi_lora_figures(dev, reps=args.multi_reps, graph=not args.no_graph)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
