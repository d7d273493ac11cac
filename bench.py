#!/usr/bin/env python3
"""Throughput of the SVDQuant W4A4 + low-rank path on one MI355X.

One step is one pass of the whole runtime path over one batch of synthetic
input already resident in HBM:
    fc1  4608 x 3072 -> 12288, rank 32: quantise + low-rank down (kernel 1),
         INT4 GEMM + low-rank up + bias + tanh-GELU, whose epilogue rounds to
         bf16 and quantises fc2's input (codes, scales, low-rank down) (kernel 2)
    fc2  4608 x 12288 -> 3072, rank 32: kernel 2 on that input
    AWQ  W4A16 modulation projection 1 x 3072 -> 18432 (kernel 3)
The same step with fc1's output stored and fc2 quantised by its own kernel 1
is timed too (`unfused_pair`).
The offline steps (smoothing, SVD split, residual quantisation, AWQ
quantisation) run once before timing, through the library's host code.

value = 2 * (2 M N K) of the two W4A4 layers / step time, in TOPS, where the
step time comes from K uninstrumented steps (an event between two kernels
costs a few microseconds of its own).  A second pass of K steps with events
recorded on the launch stream between kernels gives each kernel's duration;
the dominant kernel (the W4A4 GEMM) is reported against the int8 MFMA peak.
Input and weight buffers rotate over several copies so the 256 MB
Infinity Cache cannot hold a step's working set between uses.
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

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, 256 CU x 2.4 GHz x 8192 ops/clk
PEAK_HBM_GBS = 8000.0
PEAK_FP4_TOPS = 10100.0     # MI355X dense FP4 MFMA
PEAK_FP6_TOPS = 10100.0     # MI355X dense FP6 MFMA (the instruction the INT4 GEMM runs on)
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "w4a4_rank_corrected_smooth_amd", "csrc", "device.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def cpu_baseline(sample_rows_fc1=3072, sample_rows_fc2=1536, min_seconds=10.0, max_runs=40):
    """The oracle as it stands, timed on the host cores over a bounded sample:
    every token row of both layers, for a slice of each layer's output
    channels (prepare untimed).  The sample's forward is repeated until at
    least ``min_seconds`` of CPU work have been timed."""
    import numpy as np
    import synth
    from oracle import svdquant as O
    from oracle import glue as OG
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info()) or 1
    except Exception:
        cores = len(os.sched_getaffinity(0))
    fc1, W2, b2 = synth.mlp_cases()
    M, K1, K2 = fc1.M, fc1.K, W2.shape[1]
    ref1 = O.prepare(fc1.W[:sample_rows_fc1], fc1.calib_absmax(), fc1.bias[:sample_rows_fc1], 32)
    rng = np.random.default_rng(12)
    pre = synth.f32_to_bf16_bits(rng.standard_normal((M, K2), dtype=np.float32))
    X2 = O.bf16_bits_of(OG.gelu_tanh_bf16(O.bf16_values(pre)))
    ref2 = O.prepare(W2[:sample_rows_fc2], O.calibration_absmax(O.bf16_values(X2[:64])),
                     b2[:sample_rows_fc2], 32)
    runs, t = 0, 0.0
    while runs < max_runs and (runs == 0 or t < min_seconds):
        t0 = time.perf_counter()
        O.forward(ref1, fc1.X)
        O.forward(ref2, X2)
        t += time.perf_counter() - t0
        runs += 1
    ops = runs * (2.0 * M * sample_rows_fc1 * K1 + 2.0 * M * sample_rows_fc2 * K2)
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": (f"oracle forward (activation quantisation, low-rank down, float64 "
                       f"group-scaled GEMM, low-rank up, bias) over all {M} tokens for "
                       f"{sample_rows_fc1} of fc1's 12288 and {sample_rows_fc2} of fc2's 3072 "
                       f"output channels, repeated {runs} times: {t:.1f} s"),
            "seconds": round(t, 2)}


# ------------------------------------------------------------------ profiles
K2_NAME = "k2_w4a4_gemm"


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    """The one *suffix file under d; a directory holding the output of more
    than one profiler run is refused, so runs are never mixed."""
    hits = sorted(os.path.join(root, f) for root, _, files in os.walk(d) for f in files if f.endswith(suffix))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    if len(hits) > 1:
        raise RuntimeError(f"{len(hits)} *{suffix} files under {d} (output of several runs): {hits}")
    return hits[0]


def _short(name):
    return name.split("(")[0].replace("void ", "")


def summarize_profiles(trace_dir, fetch_dir, write_dir, out_dir, command, run_log=None):
    """CPU-only: turn rocprofv3 output (one --kernel-trace --stats run, one
    FETCH_SIZE pass, one WRITE_SIZE pass, all of ``bench.py
    --calibration-copy``) into the text summaries kept under profiles/ and
    the per-launch HBM traffic of the GEMM kernel."""
    import numpy as np
    stats = _read_csv(_find(trace_dir, "kernel_stats.csv"))
    lines = ["# Kernel durations, Flux MLP pair 4608x3072x12288 r32 + AWQ 1x3072x18432",
             "", "Command (rocprofv3 --kernel-trace --stats):", "", "```", command["trace"], "```", "",
             "| kernel | calls | average us | min us | max us | share |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in stats:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    # The per-launch trace: the last `last` launches of each kernel are the
    # bench's instrumented pass, whose event-timed mean the JSON reports
    # (earlier launches include the warm-up while clocks settle).
    last = 50
    trace = _read_csv(_find(trace_dir, "kernel_trace.csv"))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = {}
    for r in trace:
        dur.setdefault(_short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", f"Mean over each kernel's last {last} launches (the bench's instrumented pass):", "",
              "| kernel | launches | mean us (last) |", "|---|---:|---:|"]
    for k, v in dur.items():
        if len(v) >= last:
            lines.append(f"| `{k}` | {len(v)} | {float(np.mean(v[-last:])):.2f} |")
    k2_last = [float(np.mean(v[-last:])) for k, v in dur.items() if K2_NAME in k and len(v) >= last]
    if k2_last:
        lines += ["", f"{K2_NAME}: mean of its kernels' last-{last} means {float(np.mean(k2_last)):.2f} us "
                  "(compare `roofline.avg_launch_us` of the same run)."]
    if run_log:
        # the JSON line the profiled bench run printed
        js = [ln for ln in open(run_log) if ln.startswith("{")]
        if js:
            d = json.loads(js[-1])
            lines += [f"The profiled run's own JSON: `roofline.avg_launch_us` = {d['roofline']['avg_launch_us']} us, "
                      f"`kernels_us` = {d['kernels_us']}."]
    with open(os.path.join(out_dir, "kernels_flux_mlp_pair.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(d, counter):
        rows = [r for r in _read_csv(_find(d, "counter_collection.csv")) if r["Counter_Name"] == counter]
        by = {}
        for r in rows:
            by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return by
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_name = [k for k in fetch if "neg" in k.lower()]
    if not copy_name:
        raise RuntimeError("the calibration copy kernel is missing from the FETCH_SIZE pass")
    copy_bytes = CALIBRATION_BYTES
    f_fac = float(np.median(fetch[copy_name[0]])) / copy_bytes
    w_fac = float(np.median(write[copy_name[0]])) / copy_bytes
    out = {"source_hash": source_hash(), "fetch_factor": f_fac, "write_factor": w_fac,
           "calibration": f"elementwise negate of {copy_bytes} bytes float32 into a second buffer",
           "kernels": {}}
    tl = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated)", "",
          "Commands (one pass per counter):", "", "```", command["fetch"], command["write"], "```", "",
          f"Calibration: elementwise negate of {copy_bytes / 2**20:.0f} MiB float32 reads and writes "
          f"{copy_bytes / 2**20:.0f} MiB; the counters read {f_fac:.3f}x (fetch) and {w_fac:.3f}x (write) "
          "of that, and every figure below is divided by those factors.", "",
          "| kernel | launches | fetch MB | write MB | total MB |", "|---|---:|---:|---:|---:|"]
    for k in fetch:
        if k not in write:
            continue
        fb = float(np.mean(fetch[k])) / f_fac
        wb = float(np.mean(write[k])) / w_fac
        out["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "launches": len(fetch[k])}
        tl.append(f"| `{k[:90]}` | {len(fetch[k])} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} |")
    k2 = [v for k, v in out["kernels"].items() if K2_NAME in k]
    if k2:
        out["bytes_per_launch"] = float(np.mean([v["fetch_bytes"] + v["write_bytes"] for v in k2]))
        tl += ["", f"{K2_NAME} mean over its launches: {out['bytes_per_launch'] / 1e6:.1f} MB per launch."]
    with open(os.path.join(out_dir, "hbm_traffic_flux_mlp_pair.md"), "w") as f:
        f.write("\n".join(tl) + "\n")
    with open(os.path.join(out_dir, "k2_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines + [""] + tl))


CALIBRATION_BYTES = 256 << 20


SQ_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU")
# a second pass: where the wavefronts' cycles go (waits, issue, LDS)
SQ_COUNTERS_MEM = ("GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
                   "SQ_ACTIVE_INST_ANY", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT")


def summarize_trace(trace_dir, out_path, title, command, json_path=None, note=""):
    """CPU only: a rocprofv3 --kernel-trace --stats run as a text summary
    (per-kernel calls and durations), with the command that made it and, if
    given, the JSON lines the traced run printed."""
    lines = [f"# {title}", ""]
    if note:
        lines += [note, ""]
    lines += ["Command:", "", "```", command, "```", ""]
    if trace_dir:
        stats = _read_csv(_find(trace_dir, "kernel_stats.csv"))
        lines += ["| kernel | calls | average us | min us | max us | share |", "|---|---:|---:|---:|---:|---:|"]
        for r in stats:
            lines.append(f"| `{_short(r['Name'])[:80]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
        lines.append("")
    if json_path:
        js = [ln.strip() for ln in open(json_path) if ln.startswith("{")]
        if js:
            lines += ["The run's own output:", "", "```"] + js + ["```"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_mfma(jsonl, out_path, command):
    """CPU only: the --mfma-peak lines as a table (rate against the published
    dense peak of each instruction)."""
    allrows = [json.loads(l) for l in open(jsonl) if l.startswith("{")]
    rows = [r for r in allrows if "mfma" in r]
    mixes = {r["kind"]: r for r in allrows if "mix" in r}
    lines = ["# Achievable matrix-instruction rates (registers only)", "",
             "svdq_measure_mfma: 512 workgroups of 256 threads (two per CU, two wavefronts per SIMD), every "
             "wavefront four independent accumulation chains of `iters` instructions of one kind; one launch "
             "timed with events after three warm-up launches, median of five.  Rate = instructions x "
             "operations per instruction / time.  The shader clock read after a launch this short is not "
             "reliable, so no cycle count is derived from it.", "",
             "Command:", "", "```", command, "```", "",
             "| instruction | ms per launch | rate (T ops/s) | published dense peak | fraction |",
             "|---|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| {r['mfma']} | {r['ms']:.3f} | {r['rate_tops']:.0f} | {r['peak_tops']:.0f} | "
                     f"{r['frac_of_peak']:.1%} |")
    if mixes:
        fp6 = [r for r in rows if r["mfma"].startswith("fp6")]
        lines += ["", "## Instruction mixes", "",
                  "Same launch shape; one slot per chain and iteration.  Time per slot is what one SIMD spends on "
                  "it with two wavefronts resident.", "",
                  "| mix | ms per launch | ns per slot per SIMD |", "|---|---:|---:|"]
        for k in sorted(mixes):
            lines.append(f"| {mixes[k]['mix']} | {mixes[k]['ms']:.3f} | {mixes[k]['ns_per_slot_per_simd']:.2f} |")
        if fp6 and 5 in mixes and 6 in mixes:
            a, b = fp6[0]["ns_per_instruction_per_simd"], mixes[6]["ns_per_slot_per_simd"]
            c = mixes[5]["ns_per_slot_per_simd"]
            lines += ["", f"An fp6 instruction alone takes {a:.2f} ns and 16 FMAs alone {b:.2f} ns; together, on "
                      f"independent registers, {c:.2f} ns, {c / (a + b):.0%} of their sum: on a SIMD the vector "
                      "ALU runs beside the matrix core for only a small part of the time, so the GEMM's time per "
                      "group is close to the sum of its matrix and vector instructions."]
        x8 = [r for r in rows if r["mfma"].startswith("bf16 32x32x8")]
        if 7 in mixes and fp6 and x8 and 6 in mixes:
            parts = (x8[0]["ns_per_instruction_per_simd"] + fp6[0]["ns_per_instruction_per_simd"]
                     + mixes[6]["ns_per_slot_per_simd"])
            lines += ["", f"The GEMM's step takes {mixes[7]['ns_per_slot_per_simd']:.2f} ns against {parts:.2f} ns "
                      f"for its three parts alone ({mixes[7]['ns_per_slot_per_simd'] / parts:.0%})."]
        if 7 in mixes:
            g = 8 * mixes[7]["ns_per_slot_per_simd"]
            # fc2 at 4608 x 3072, K = 12288: 36 x 12 tiles of 128 x 256 on 256 CUs x 2 slots; the busiest
            # CU holds two workgroups, so each of its SIMDs runs 2 x 192 wavefront-groups
            lines += ["", f"The GEMM's step for one tile: {mixes[7]['ns_per_slot_per_simd']:.2f} ns; a wavefront's "
                      f"group (8 tiles) {g:.0f} ns of SIMD time.  At fc2 (4608 x 3072, K = 12288: 432 tiles of "
                      f"128 x 256, at most two workgroups on a CU, 2 x 192 wavefront-groups per SIMD) that is "
                      f"{384 * g / 1e3:.0f} us for the main loop alone, with no wait, prologue or epilogue."]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_floor(trace_dir, jsonl, out_path, command):
    """CPU only: the streaming read and copy kernels of ``--hbm-floor`` from a
    rocprofv3 kernel trace, by case and grid: each back-to-back series is a
    run of launches with one grid size, in the order the mode issues them;
    the mean of a series' last 150 launches (the five timed batches of 30)
    gives the kernel's own duration and rate, free of launch gaps."""
    import numpy as np
    cases = [json.loads(l) for l in open(jsonl) if l.startswith("{")]
    rows = sorted(_read_csv(_find(trace_dir, "kernel_trace.csv")), key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    for r in rows:
        if "stream_probe" not in r["Kernel_Name"]:
            continue
        g = int(r["Grid_Size_X"]) // 256
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if runs and runs[-1][0] == g:
            runs[-1][1].append(d)
        else:
            runs.append((g, [d]))
    lines = ["# Practical HBM floor at the bandwidth-bound kernels' sizes", "",
             "A plain streaming read (16 loads of 16 bytes in flight per lane, nontemporal) and a plain copy of "
             "the quantiser's input (4608 x 3072 and 4608 x 12288 bf16) and of the W4A16 blob (18432 x 3072), "
             "over rotating buffers larger than the 256 MB Infinity Cache.  Durations are the kernel trace's own "
             "(mean of each series' last 150 launches), so launch gaps are excluded.", "",
             "Command:", "", "```", command, "```", "",
             "| case | bytes | grid | read us | read GB/s | fraction of 8 TB/s |", "|---|---:|---:|---:|---:|---:|"]
    i = 0
    for c in cases:
        grids = sorted(int(k) for k in c["read_gbs_by_grid"])
        for g in grids + ["copy"]:
            if i >= len(runs):
                break
            gg, ds = runs[i]
            i += 1
            us = float(np.mean(ds[-150:]))
            nb = c["bytes"] * (2 if g == "copy" else 1)
            label = f"{c['kernel_grid']} (copy)" if g == "copy" else str(g)
            mark = " (kernel's grid)" if g == c["kernel_grid"] else ""
            lines.append(f"| {c['hbm_floor']} | {c['bytes']} | {label}{mark} | {us:.2f} | {nb / us / 1e3:.0f} | "
                         f"{nb / us / 1e3 / PEAK_HBM_GBS:.1%} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_means(pmc_dir, counters):
    """Per-kernel means of a rocprofv3 --pmc pass (the library's kernels
    only) and each kernel's dispatch durations (us)."""
    import csv
    import glob
    from collections import defaultdict
    import numpy as np
    path = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)[0]
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        if not any(k in name for k in ("k1_quantize", "k2_w4a4", "k3_awq")):
            continue
        vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        durs[name][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = {}
    for name in sorted(vals):
        v = {c: float(np.mean(vals[name][c])) for c in counters if vals[name][c]}
        if len(v) == len(counters):
            out[name] = (v, len(durs[name]), float(np.mean(list(durs[name].values()))))
    return out


def summarize_counters(pmc_dir, out_path, command):
    """Per-kernel shader counters (one rocprofv3 --pmc pass of the default
    profile command), averaged over each kernel's dispatches, with the clock
    and the vector-ALU and matrix-pipe occupancy they imply."""
    simds, xcds = 1024, 8
    lines = ["# Shader counters per kernel, Flux MLP pair 4608x3072x12288 r32 + AWQ 1x3072x18432", "",
             "Command:", "", "```", command, "```", "",
             "Means over each kernel's dispatches.  cycles = GRBM_GUI_ACTIVE / 8 XCDs (the GPU's busy "
             "cycles while the kernel runs; for kernels of a few microseconds they include the counter "
             "pass's own start-up).  VALU busy = (SQ_INSTS_VALU - SQ_INSTS_MFMA) x 4 cycles (a wave64 "
             "vector instruction holds its SIMD 4 cycles) / (1024 SIMDs x cycles); matrix busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles).  Durations come from the counter pass, "
             "which runs slower than a plain trace.", "",
             "| kernel | dispatches | us | cycles | " + " | ".join(SQ_COUNTERS[1:]) + " | VALU busy | matrix busy |",
             "|---|---:|---:|---:|" + "---:|" * (len(SQ_COUNTERS) - 1) + "---:|---:|"]
    for name, (v, n, d) in _counter_means(pmc_dir, SQ_COUNTERS).items():
        cyc = v["GRBM_GUI_ACTIVE"] / xcds
        valu = (v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"]) * 4 / (simds * cyc)
        mfma = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cyc)
        lines.append(f"| `{name}` | {n} | {d:.1f} | {cyc:.4g} | " +
                     " | ".join(f"{v[c]:.4g}" for c in SQ_COUNTERS[1:]) + f" | {valu:.0%} | {mfma:.0%} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters_mem(pmc_dir, out_path, command):
    """The second counter pass: the share of the wavefronts' cycles spent
    waiting on s_waitcnt (SQ_WAIT_ANY), waiting for an instruction to issue
    (SQ_WAIT_INST_ANY) and issuing (SQ_ACTIVE_INST_ANY), all against
    SQ_WAVE_CYCLES, and the LDS instruction and bank-conflict counts."""
    xcds = 8
    lines = ["# Where the wavefronts' cycles go, Flux MLP pair 4608x3072x12288 r32 + AWQ 1x3072x18432", "",
             "Command:", "", "```", command, "```", "",
             "Means over each kernel's dispatches.  The three shares are of SQ_WAVE_CYCLES (the cycles "
             "summed over resident wavefronts): SQ_WAIT_ANY counts cycles a wavefront waits on a counter "
             "(s_waitcnt: memory, LDS), SQ_WAIT_INST_ANY cycles it waits for its next instruction to "
             "issue (a dependency, a busy pipe, the barrier), SQ_ACTIVE_INST_ANY cycles it issues; the "
             "LDS wait share is SQ_WAIT_INST_LDS of the same.  Conflicts per LDS instruction = "
             "SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS.  Durations come from the counter pass.", "",
             "| kernel | dispatches | us | cycles | " + " | ".join(SQ_COUNTERS_MEM[1:]) +
             " | waiting on counters | waiting to issue | issuing | LDS wait share | conflicts per LDS instr |",
             "|---|---:|---:|---:|" + "---:|" * (len(SQ_COUNTERS_MEM) - 1) + "---:|---:|---:|---:|---:|"]
    for name, (v, n, d) in _counter_means(pmc_dir, SQ_COUNTERS_MEM).items():
        cyc = v["GRBM_GUI_ACTIVE"] / xcds
        wc = max(v["SQ_WAVE_CYCLES"], 1.0)
        lines.append(f"| `{name}` | {n} | {d:.1f} | {cyc:.4g} | " +
                     " | ".join(f"{v[c]:.4g}" for c in SQ_COUNTERS_MEM[1:]) +
                     f" | {v['SQ_WAIT_ANY'] / wc:.0%} | {v['SQ_WAIT_INST_ANY'] / wc:.0%} |"
                     f" {v['SQ_ACTIVE_INST_ANY'] / wc:.0%} | {v['SQ_WAIT_INST_LDS'] / wc:.1%} |"
                     f" {v['SQ_LDS_BANK_CONFLICT'] / max(v['SQ_INSTS_LDS'], 1.0):.3f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_configs(trace_dir, sweep_jsonl, out_path, command):
    """Exact per-configuration kernel durations from a rocprofv3 kernel trace
    of ``bench.py --configs``: the sweep launches each timed kernel 8 + steps
    + 5 x 24 times in a row, in a fixed order of configurations, so the
    trace's runs of one kernel split into those series; the last 120 launches
    of each are the back-to-back ones."""
    import csv
    import glob
    import numpy as np
    cfgs = [json.loads(l) for l in open(sweep_jsonl) if l.startswith("{")]
    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    for r in rows:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if "k2_split_sum" in name and runs and "k2_w4a4" in runs[-1][0]:
            runs[-1][1][-1] += d          # a K-split GEMM's second kernel: one launch of the layer's K2
            continue
        if runs and runs[-1][0] == name:
            runs[-1][1].append(d)
        else:
            runs.append((name, [d]))
    per = 8 + 50 + 5 * 24
    series = []      # (kernel, durations of one timed series)
    for name, ds in runs:
        if not any(k in name for k in ("k1_quantize", "k2_w4a4", "k3_awq")) or len(ds) < per:
            continue
        n = len(ds) // per
        for i in range(n):
            series.append((name, ds[len(ds) - (n - i) * per: len(ds) - (n - i - 1) * per]))
    lines = ["# Kernel durations per configuration (rocprofv3 kernel trace)", "",
             "Command:", "", "```", command, "```", "",
             "Each kernel runs as its own series (8 warm-up launches, 50 launches between events, "
             "then 5 x 24 back to back) over rotating buffer sets; durations below are the trace's "
             "own, over the 120 back-to-back launches (a K-split GEMM counts with its partial-sum "
             "kernel). Rates use the algorithmic work of each "
             "kernel (K2: 2MNK int ops; K1: X + 1/lambda + L1s + codes + scales + D bytes; "
             "K3: codes + scales/zeros + x + y bytes).", "",
             "K2's fraction is of its own instruction's peak (fp6 for INT4 codes, fp4 for MXFP4: 10.1 "
             "POP/s each), with the int8 peak (5.0 POP/s) of the metric beside the rate; K1 and K3 are "
             "against 8 TB/s.  A layer row gives 2MNK over the sum of its K1 and K2 medians.", "",
             "| configuration | kernel | median us | p10 us | p90 us | rate | fraction of peak |",
             "|---|---|---:|---:|---:|---:|---:|"]
    si = 0
    for c in cfgs:
        if "k3" in c:
            kinds = [("K3", "k3_awq")]
        else:
            kinds = [("K1", "k1_quantize"), ("K2", "k2_w4a4")]
        meds = {}
        for label, key in kinds:
            while si < len(series) and key not in series[si][0]:
                si += 1
            if si >= len(series):
                break
            name, ds = series[si]
            si += 1
            b2b = np.array(ds[-120:])
            med = float(np.median(b2b))
            meds[label] = med
            M, N, K = c["M"], c["N"], c["K"]
            if label == "K2":
                rate = 2.0 * M * N * K / med / 1e6
                pk = PEAK_FP4_TOPS if c.get("format") == "mxfp4" else PEAK_FP6_TOPS
                txt, frac = f"{rate:.0f} TOPS ({rate / PEAK_INT8_TOPS:.1%} of int8)", rate / pk
            elif label == "K1":
                r = c["rank"]
                b = 2 * M * K + 4 * K + 2 * K * r + M * K // 2 + 4 * M * (K // 64) + 4 * M * r
                rate = b / med / 1e3
                txt, frac = f"{rate:.0f} GB/s", rate / PEAK_HBM_GBS
            else:
                b = N * K // 2 + N * (K // 64) * 4 + M * K * 2 + M * N * 2
                rate = b / med / 1e3
                txt, frac = f"{rate:.0f} GB/s", rate / PEAK_HBM_GBS
            lines.append(f"| {c['config']} ({M}x{K}->{N}) | `{name}` | {med:.2f} | "
                         f"{np.percentile(b2b, 10):.2f} | {np.percentile(b2b, 90):.2f} | {txt} | {frac:.1%} |")
        if "K1" in meds and "K2" in meds:
            # the layer: 2MNK over the two kernels' median durations together
            M, N, K = c["M"], c["N"], c["K"]
            t = meds["K1"] + meds["K2"]
            rate = 2.0 * M * N * K / t / 1e6
            pk = PEAK_FP4_TOPS if c.get("format") == "mxfp4" else PEAK_FP6_TOPS
            lines.append(f"| {c['config']} ({M}x{K}->{N}) | layer (K1 + K2) | {t:.2f} | | | "
                         f"{rate:.0f} TOPS ({rate / PEAK_INT8_TOPS:.1%} of int8) | {rate / pk:.1%} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mx_pair(args, S, fc1, W2, b2, ax2, X, R, dev, stream):
    """The MLP pair in the FP4 (MXFP4) form of the path, on the same inputs:
    fc1 quantise, fc1 GEMM + GELU (bf16 out), fc2 quantise, fc2 GEMM, timed
    like the step (uninstrumented steps for the rate, a pass with events
    between kernels for each kernel's duration).  Reported beside the INT4
    headline, not instead of it."""
    import numpy as np
    import torch
    log("MXFP4 form: preparing fc1 and fc2 on the host")
    m1 = [S.MxLinear(S.mx_prepare_weights(fc1.W, fc1.calib_absmax(), fc1.bias, 32), dev) for _ in range(R)]
    m2 = [S.MxLinear(S.mx_prepare_weights(W2, ax2, b2, 32), dev) for _ in range(R)]
    M, N1, K1 = fc1.M, fc1.N, fc1.K
    w1 = [m1[0].new_workspace(M) for _ in range(R)]
    w2 = [m2[0].new_workspace(M) for _ in range(R)]
    Y1 = [torch.empty((M, N1), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    Y2 = [torch.empty((M, K1), dtype=torch.bfloat16, device=dev) for _ in range(R)]

    def step(i, ev=None):
        k = i % R

        def mark(j):
            if ev:
                ev[j].record(stream)
        mark(0)
        S.mx_linear_quantize(m1[k], X[k], w1[k])
        mark(1)
        S.mx_linear_gemm(m1[k], M, Y1[k], w1[k], gelu=True)
        mark(2)
        S.mx_linear_quantize(m2[k], Y1[k], w2[k])
        mark(3)
        S.mx_linear_gemm(m2[k], M, Y2[k], w2[k])
        mark(4)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    settle(step, 0.1)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    names = ["fc1_quantize", "fc1_gemm_gelu", "fc2_quantize", "fc2_gemm"]
    us = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs])) for j, n in enumerate(names)}
    ops = 2.0 * M * N1 * K1
    k2 = 0.5 * (us["fc1_gemm_gelu"] + us["fc2_gemm"])
    del m1, m2, w1, w2, Y1, Y2
    torch.cuda.empty_cache()
    return {"format": "mxfp4 (OCP MX: E2M1 codes, E8M0 scale per 32)",
            "ms_per_step": round(wall / args.steps * 1e3, 4),
            "value": round(2 * ops / (wall / args.steps) / 1e12, 2), "unit": "TOPS",
            "kernels_us": {n: round(v, 2) for n, v in us.items()},
            "k2_avg_us": round(k2, 2), "k2_tops": round(ops / k2 / 1e6, 1),
            "k2_frac_int8": round(ops / k2 / 1e6 / PEAK_INT8_TOPS, 4),
            "k2_frac_fp4": round(ops / k2 / 1e6 / PEAK_FP4_TOPS, 4)}


def config_sweep(args):
    """Per-configuration kernel timings (not the one-line contract): for each
    W4A4 configuration, the quantiser (kernel 1) and the GEMM (kernel 2) are
    timed apart, and the AWQ kernel at M = 1, 2, 4, 8, 16.  Each kernel is
    timed two ways over rotating buffer sets (enough copies that a series
    touches more than the 256 MB Infinity Cache): per launch between HIP
    events (median, p10, p90; each includes a few microseconds of event
    overhead), and as the mean of 24 launches back to back between two
    events.  One JSON line per configuration; a rocprofv3 kernel trace of
    this mode gives the exact durations."""
    import numpy as np
    import torch
    import synth
    import w4a4_rank_corrected_smooth_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S.device_check()
    stream = torch.cuda.current_stream(dev)
    reps, batch = args.steps, 24

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def nsets(bytes_per_set):
        return int(min(32, max(3, -(-640e6 // bytes_per_set))))

    def timed(fn, R):
        for i in range(8):
            fn(i % R)
        torch.cuda.synchronize()
        per = []
        for i in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(i % R)
            e1.record(stream)
            per.append((e0, e1))
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) * 1e3 for a, b in per])
        b2b = []
        for r in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(batch):
                fn(i % R)
            e1.record(stream)
            torch.cuda.synchronize()
            b2b.append(e0.elapsed_time(e1) * 1e3 / batch)
        return {"median_us": round(float(np.median(t)), 2), "p10_us": round(float(np.percentile(t, 10)), 2),
                "p90_us": round(float(np.percentile(t, 90)), 2),
                "back_to_back_us": round(float(np.median(b2b)), 2)}

    def w4a4(name, M, N, K, r, hw, Xbits, gelu, mx=False, extra=None):
        R = nsets(2 * M * K + M * N * 2 + N * K // 2 + S.workspace_bytes(M, N, K, r))
        log(f"{name}: {R} buffer sets")
        Ls = [(S.MxLinear if mx else S.Linear)(hw, dev) for _ in range(R)]
        Xs = [dev_bf16(Xbits) if isinstance(Xbits, np.ndarray) else Xbits.clone() for _ in range(R)]
        ws = [Ls[0].new_workspace(M) for _ in range(R)]
        Ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
        quant = S.mx_linear_quantize if mx else S.linear_quantize
        gemm = S.mx_linear_gemm if mx else S.linear_gemm
        for k in range(R):
            quant(Ls[k], Xs[k], ws[k])
        k1 = timed(lambda k: quant(Ls[k], Xs[k], ws[k]), R)
        k2 = timed(lambda k: gemm(Ls[k], M, Ys[k], ws[k], gelu=gelu), R)
        ops = 2.0 * M * N * K
        k1_bytes = 2 * M * K + 4 * K + 2 * K * r + M * K // 2 + 4 * M * (K // 64) + 4 * M * r
        t1, t2 = k1["back_to_back_us"], k2["back_to_back_us"]
        out = {"config": name, "M": M, "N": N, "K": K, "rank": r, "gelu": gelu, "sets": R,
               "k1": k1, "k2": k2, "format": "mxfp4" if mx else "int4",
               "k2_tops": round(ops / t2 / 1e6, 1), "k2_frac_int8": round(ops / t2 / 1e6 / PEAK_INT8_TOPS, 4),
               "k1_gbs": round(k1_bytes / t1 / 1e3, 1), "k1_frac_hbm": round(k1_bytes / t1 / 1e3 / PEAK_HBM_GBS, 4),
               "layer_tops": round(ops / (t1 + t2) / 1e6, 1),
               "lowrank_gflop": round(2.0 * M * (K + N) * r / 1e9, 2)}
        out.update(extra or {})
        print(json.dumps(out), flush=True)
        del Ls, Xs, ws, Ys
        torch.cuda.empty_cache()

    c = synth.tiny_case()
    w4a4("tiny", c.M, c.N, c.K, 16, S.prepare_weights(c.W, c.calib_absmax(), c.bias, 16), c.X, False)
    c = synth.qkv_case()
    log("preparing QKV on the host")
    w4a4("qkv", c.M, c.N, c.K, 32, S.prepare_weights(c.W, c.calib_absmax(), c.bias, 32), c.X, False)
    fc1, W2, b2 = synth.mlp_cases()
    log("preparing fc1 on the host")
    hw1 = S.prepare_weights(fc1.W, fc1.calib_absmax(), fc1.bias, 32)
    w4a4("mlp_fc1_gelu", fc1.M, fc1.N, fc1.K, 32, hw1, fc1.X, True)
    # a user LoRA of rank 32 carried by the branch (merged rank 64)
    A, B = synth.lora_factors(5, fc1.N, fc1.K, 32)
    t0 = time.perf_counter()
    hwl = S.merge_lora(hw1, A, B, 1.0)
    merge_s = time.perf_counter() - t0
    w4a4("mlp_fc1_gelu_lora32", fc1.M, fc1.N, fc1.K, 64, hwl, fc1.X, True,
         extra={"lora_rank": 32, "merge_s": round(merge_s, 4)})
    del hwl
    L1 = S.Linear(hw1, dev)
    Y1 = S.linear_forward(L1, dev_bf16(fc1.X), out_dtype=torch.bfloat16, gelu=True)
    torch.cuda.synchronize()
    ax2 = S.calibration_absmax(Y1[:64].cpu().view(torch.int16).numpy().view(np.uint16))
    log("preparing fc2 on the host")
    hw2 = S.prepare_weights(W2, ax2, b2, 32)
    del L1
    w4a4("mlp_fc2", fc1.M, fc1.K, fc1.N, 32, hw2, Y1, False)
    del Y1
    c = synth.lowres_case()
    log("preparing the low-resolution layer on the host")
    w4a4("lowres_r128", c.M, c.N, c.K, 128, S.prepare_weights(c.W, c.calib_absmax(), c.bias, 128), c.X, False)
    # the FP4 (MXFP4) form on the same layers
    c = synth.qkv_case()
    w4a4("qkv_mxfp4", c.M, c.N, c.K, 32, S.mx_prepare_weights(c.W, c.calib_absmax(), c.bias, 32), c.X,
         False, mx=True)
    w4a4("mlp_fc1_gelu_mxfp4", fc1.M, fc1.N, fc1.K, 32,
         S.mx_prepare_weights(fc1.W, fc1.calib_absmax(), fc1.bias, 32), fc1.X, True, mx=True)
    X2 = dev_bf16(np.random.default_rng(2).standard_normal((fc1.M, fc1.N), dtype=np.float32)
                  .view(np.uint32).__rshift__(16).astype(np.uint16))
    w4a4("mlp_fc2_mxfp4", fc1.M, fc1.K, fc1.N, 32, S.mx_prepare_weights(W2, None, b2, 32), X2, False, mx=True)
    del X2
    a = synth.awq_case()
    q, sc, z = S.awq_quantize_weights(a.W)
    R = nsets(a.N * a.K // 2 + a.N * (a.K // 64) * 4)
    A = [S.AwqLinear(q, sc, z, dev) for _ in range(R)]
    for M in (1, 2, 4, 8, 16):
        xs = [torch.from_numpy(np.ascontiguousarray(a.x[:M])).to(dev) for _ in range(R)]
        ys = [torch.empty((M, a.N), dtype=torch.float16, device=dev) for _ in range(R)]
        k3 = timed(lambda k: S.awq_forward(A[k], xs[k], out=ys[k]), R)
        nbytes = a.N * a.K // 2 + a.N * (a.K // 64) * 4 + M * a.K * 2 + M * a.N * 2
        t3 = k3["back_to_back_us"]
        print(json.dumps({"config": f"awq_m{M}", "M": M, "N": a.N, "K": a.K, "sets": R, "k3": k3,
                          "k3_gbs": round(nbytes / t3 / 1e3, 1),
                          "k3_frac_hbm": round(nbytes / t3 / 1e3 / PEAK_HBM_GBS, 4)}), flush=True)


def block_study(args):
    """Launch study of one transformer block's calls into the library (not
    the one-line contract): the AWQ modulation projection (1 x 3072 ->
    18432), the QKV (3072 -> 9216) and output (3072 -> 3072) projections and
    the fused MLP pair (3072 -> 12288 -> 3072), all rank 32, at 4608 and
    1024 tokens.  The same sequence runs eagerly (every call launched from
    Python through the C ABI) and as one captured HIP graph; each call is
    also timed alone between events.  One JSON line per token count.
    Attention sits between these calls in a real block and is not part of
    this library, so it is left out."""
    import numpy as np
    import torch
    import synth
    import w4a4_rank_corrected_smooth_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S.device_check()
    D, F = 3072, 12288
    log("block study: preparing QKV, output projection, fc1, fc2 and AWQ on the host")
    fc1c, W2, b2 = synth.mlp_cases()
    qc = synth.qkv_case()
    oc = synth.linear_case("out_proj", 6, 8, D, D, 32, x_outlier_frac=0.005, x_outlier_scale=50.0)
    qkv = S.Linear(S.prepare_weights(qc.W, qc.calib_absmax(), qc.bias, 32), dev)
    outp = S.Linear(S.prepare_weights(oc.W, oc.calib_absmax(), oc.bias, 32), dev)
    fc1 = S.Linear(S.prepare_weights(fc1c.W, fc1c.calib_absmax(), fc1c.bias, 32), dev)
    fc2 = S.Linear(S.prepare_weights(W2, None, b2, 32), dev)
    a = synth.awq_case()
    q, sc, z = S.awq_quantize_weights(a.W)
    awq = S.AwqLinear(q, sc, z, dev)
    x1 = torch.from_numpy(np.ascontiguousarray(a.x[:1])).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    for M in (4608, 1024):
        X = torch.from_numpy(np.ascontiguousarray(qc.X[:M]).view(np.int16)).view(torch.bfloat16).to(dev)
        mod = torch.empty(1, a.N, dtype=torch.float16, device=dev)
        Yq = torch.empty(M, 3 * D, dtype=torch.bfloat16, device=dev)
        Yo = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
        Ym = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
        wq, wo = qkv.new_workspace(M), outp.new_workspace(M)
        w1, w2 = fc1.new_workspace(M), fc2.new_workspace(M)
        calls = [("awq_mod", lambda: S.awq_forward(awq, x1, out=mod)),
                 ("qkv", lambda: S.linear_forward(qkv, X, out=Yq, workspace=wq)),
                 ("out_proj", lambda: S.linear_forward(outp, X, out=Yo, workspace=wo)),
                 ("mlp_pair", lambda: S.mlp_forward(fc1, fc2, X, out=Ym, ws1=w1, ws2=w2))]

        def block():
            for _, f in calls:
                f()

        stream = torch.cuda.current_stream(dev)
        for _ in range(10):
            block()
        torch.cuda.synchronize()
        n = args.steps
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(n):
            block()
        e1.record(stream)
        torch.cuda.synchronize()
        eager = e0.elapsed_time(e1) * 1e3 / n
        per = {}
        for name, f in calls:
            ts = []
            for _ in range(n):
                a0, a1 = ev(), ev()
                a0.record(stream)
                f()
                a1.record(stream)
                ts.append((a0, a1))
            torch.cuda.synchronize()
            per[name] = round(float(np.median([u.elapsed_time(v) * 1e3 for u, v in ts])), 2)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            block()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            block()
        for _ in range(5):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(n):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph = e0.elapsed_time(e1) * 1e3 / n
        print(json.dumps({"study": "block", "tokens": M, "calls_per_block": len(calls), "kernels_per_block": 8,
                          "eager_us": round(eager, 2), "graph_us": round(graph, 2),
                          "per_call_event_us": per, "sum_per_call_us": round(sum(per.values()), 2)}), flush=True)
        del g, X, Yq, Yo, Ym, wq, wo, w1, w2
        torch.cuda.empty_cache()


SETTLE_S = 0.3     # seconds of sustained load before any timed pass


def settle(fn, seconds):
    """Run `fn(i)` in batches until `seconds` of wall time have passed: the
    GPU takes tens of milliseconds of sustained load to reach steady clocks,
    whatever the warm-up step count."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(10):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def k2_mix_ceiling_us(step_ns, M, N, K, cus=256):
    """Main-loop floor of one GEMM launch from the measured time of its
    per-tile step (svdq_measure_mfma kind 7, SIMD time per step with two
    wavefronts resident): the busiest CU holds ceil(tiles / CUs) workgroup
    tiles, each putting one wavefront on every SIMD for K / 64 groups of 8
    steps.  Waits, prologue and epilogue are not in it."""
    tiles = -(-M // 128) * -(-N // 256)
    per_cu = -(-tiles // cus)
    return per_cu * (K // 64) * 8 * step_ns / 1e3


def measure_step_ns(S, dev, stream, iters=20000, grid=512):
    """SIMD time of the GEMM's per-tile step (kind 7), median of 5 launches."""
    import numpy as np
    import torch
    sink = torch.zeros(grid, dtype=torch.int32, device=dev)
    for _ in range(2):
        S.measure_mfma(7, iters, grid, sink)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        S.measure_mfma(7, iters, grid, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    return float(np.median(ts)) * 1e9 * 1024 / (grid * 4 * 4 * iters)


def back_to_back(fn, stream, n=30, reps=5):
    """Median over `reps` series of the mean duration of `n` launches of
    fn(i) enqueued back to back between two events (us)."""
    import numpy as np
    import torch
    settle(fn, 0.05)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / n)
    return float(np.median(ts))


def read_sclk_mhz():
    """Current shader clock from the driver's DPM table (the level marked
    '*'), or None where the file is not readable."""
    import glob
    for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(p):
                if "*" in line:
                    return int("".join(ch for ch in line.split(":")[1] if ch.isdigit()))
        except (OSError, ValueError, IndexError):
            continue
    return None


def footprint(S, layers, awq_case):
    """Device weight bytes per layer (MB): the fp6 blob this library
    uploads, the canonical INT4 form (nibble codes, fp32 scales, bf16
    factors, 1/lambda, bias) and the layer in bf16; the AWQ blob against
    fp16."""
    out = {}
    for name, N, K, r in layers:
        canon = N * K // 2 + N * (K // 64) * 4 + 2 * (K + N) * r + 4 * K + 4 * N
        out[name] = {"device_blob": round(S.device_weights_bytes(N, K, r) / 1e6, 2),
                     "int4_canonical": round(canon / 1e6, 2), "bf16": round((2 * N * K + 2 * N) / 1e6, 2)}
    N, K = awq_case.N, awq_case.K
    out["awq_mod"] = {"device_blob": round(S._lib.awq_device_weights_bytes(N, K) / 1e6, 2),
                      "fp16": round(2 * N * K / 1e6, 2)}
    return out


def branch_fusion(S, dev, stream, layers):
    """What fusing the low-rank branch saves: each layer's forward (K1 with
    the down-projection + K2 with the up-projection) against the same layer
    with the branch as two separate bf16 GEMMs and the 4-bit GEMM's fp32
    result through memory (svdq_linear_forward_unfused), both timed back to
    back over two buffer sets."""
    import torch
    out = {}
    for name, layer, Xs, gelu in layers:
        M = Xs[0].shape[0]
        Ys = [torch.empty((M, layer.N), dtype=torch.bfloat16, device=dev) for _ in Xs]
        wf = [layer.new_workspace(M) for _ in Xs]
        wu = [torch.empty(S.unfused_workspace_bytes(M, layer.N, layer.K, layer.rank), dtype=torch.uint8,
                          device=dev) for _ in Xs]
        R = len(Xs)
        fused = back_to_back(lambda i: S.linear_forward(layer, Xs[i % R], out=Ys[i % R], gelu=gelu,
                                                        workspace=wf[i % R]), stream, n=10)
        unfused = back_to_back(lambda i: S.linear_forward_unfused(layer, Xs[i % R], out=Ys[i % R], gelu=gelu,
                                                                  workspace=wu[i % R]), stream, n=10)
        out[name] = {"M": M, "N": layer.N, "K": layer.K, "rank": layer.rank, "fused_us": round(fused, 2),
                     "unfused_us": round(unfused, 2), "fusion_saves": round(1 - fused / unfused, 4)}
        del Ys, wf, wu
        torch.cuda.empty_cache()
    return out


def cpu_configs(args):
    """bench.py --cpu-configs: the oracle's forward (activation quantisation,
    low-rank down, float64 group-scaled GEMM, low-rank up, bias; AWQ: the
    dequantised GEMV) timed on the host cores for every configuration, with
    all threads and, for the tiny and the low-res configurations, one
    thread.  The layers are prepared by the library's host code (the timed
    part is the oracle's forward alone).  One JSON line per run."""
    import numpy as np
    import synth
    import w4a4_rank_corrected_smooth_amd as S
    from oracle import awq as OA
    from oracle import glue as OG
    from oracle import svdquant as O
    from threadpoolctl import threadpool_limits, threadpool_info
    all_threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) or 1

    def ref_of(hw):
        return dict(N=hw.N, K=hw.K, rank=hw.rank, iota=hw.inv_lambda.astype(np.float32),
                    L1s=O.bf16_values(hw.l1s), L2b=O.bf16_values(hw.l2), qW=O.unpack_int4(hw.qweight),
                    sW=hw.wscales.astype(np.float32), bias=hw.bias.astype(np.float64))

    def timed(fn, min_s=1.0, max_runs=20):
        fn()
        runs, t = 0, 0.0
        while runs < max_runs and (runs == 0 or t < min_s):
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            runs += 1
        return t / runs

    def report(name, ops, fn, threads):
        with threadpool_limits(limits=threads):
            sec = timed(fn)
        print(json.dumps({"cpu_oracle": name, "threads": threads, "seconds": round(sec, 4),
                          "gops": round(ops / sec / 1e9, 2)}), flush=True)

    c = synth.tiny_case()
    ref = ref_of(S.prepare_weights(c.W, c.calib_absmax(), c.bias, 16))
    for th in (all_threads, 1):
        report("tiny_256x512x512_r16", 2.0 * c.M * c.N * c.K, lambda: O.forward(ref, c.X), th)
    c = synth.qkv_case()
    ref = ref_of(S.prepare_weights(c.W, c.calib_absmax(), c.bias, 32))
    report("qkv_4608x3072x9216_r32", 2.0 * c.M * c.N * c.K, lambda: O.forward(ref, c.X), all_threads)
    del ref
    fc1, W2, b2 = synth.mlp_cases()
    ref1 = ref_of(S.prepare_weights(fc1.W, fc1.calib_absmax(), fc1.bias, 32))
    report("mlp_fc1_4608x3072x12288_r32", 2.0 * fc1.M * fc1.N * fc1.K, lambda: O.forward(ref1, fc1.X), all_threads)
    rng = np.random.default_rng(12)
    X2 = O.bf16_bits_of(OG.gelu_tanh_bf16(O.bf16_values(
        synth.f32_to_bf16_bits(rng.standard_normal((fc1.M, fc1.N), dtype=np.float32)))))
    del ref1
    ref2 = ref_of(S.prepare_weights(W2, O.calibration_absmax(O.bf16_values(X2[:64])), b2, 32))
    report("mlp_fc2_4608x12288x3072_r32", 2.0 * fc1.M * fc1.N * fc1.K, lambda: O.forward(ref2, X2), all_threads)
    del ref2, X2
    c = synth.lowres_case()
    ref = ref_of(S.prepare_weights(c.W, c.calib_absmax(), c.bias, 128))
    for th in (all_threads, 1):
        report("lowres_1024x3072x3072_r128", 2.0 * c.M * c.N * c.K, lambda: O.forward(ref, c.X), th)
    a = synth.awq_case()
    q, sc, z = OA.quantize(a.W)
    for M in (1, 16):
        report(f"awq_m{M}_{M}x3072x18432", 2.0 * M * a.N * a.K, lambda: OA.forward(a.x[:M], q, sc, z), all_threads)


def branch_ablation_mode(args):
    """bench.py --branch-ablation: only the fused-against-unfused branch
    timings (QKV, fc1 + GELU, fc2, low-res rank 128), one JSON line; under a
    kernel trace it gives each unfused kernel's duration."""
    import numpy as np
    import torch
    import synth
    import w4a4_rank_corrected_smooth_amd as S
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S.device_check()
    stream = torch.cuda.current_stream(dev)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    log("preparing QKV, fc1, fc2 and the low-res layer on the host")
    qc, lc = synth.qkv_case(), synth.lowres_case()
    fc1, W2, b2 = synth.mlp_cases()
    L1 = S.Linear(S.prepare_weights(fc1.W, fc1.calib_absmax(), fc1.bias, 32), dev)
    x1 = [dev_bf16(fc1.X) for _ in range(2)]
    y1 = S.linear_forward(L1, x1[0], out_dtype=torch.bfloat16, gelu=True)
    torch.cuda.synchronize()
    ax2 = S.calibration_absmax(y1[:64].cpu().view(torch.int16).numpy().view(np.uint16))
    L2 = S.Linear(S.prepare_weights(W2, ax2, b2, 32), dev)
    Lq = S.Linear(S.prepare_weights(qc.W, qc.calib_absmax(), qc.bias, 32), dev)
    Ll = S.Linear(S.prepare_weights(lc.W, lc.calib_absmax(), lc.bias, 128), dev)
    res = branch_fusion(S, dev, stream, [("qkv", Lq, [dev_bf16(qc.X) for _ in range(2)], False),
                                         ("fc1_gelu", L1, x1, True), ("fc2", L2, [y1, y1.clone()], False),
                                         ("lowres_r128", Ll, [dev_bf16(lc.X) for _ in range(2)], False)])
    print(json.dumps({"study": "branch_fusion", "layers": res}), flush=True)


def mfma_peak(args):
    """Achievable issue rate of each matrix instruction the path uses, in
    registers (svdq_measure_mfma): 512 workgroups (two per CU, so two
    wavefronts per SIMD), each wavefront four independent chains; the
    launch is timed with events after a warm-up, median of 5.  One JSON line
    per instruction: the rate, its published dense peak, and the time one
    SIMD spends per instruction (the shader clock read after a launch this
    short is not reliable, so no cycle count is derived).  Then one line per
    instruction mix (an fp6 instruction with 16 independent FMAs, the FMAs
    alone, the GEMM's per-tile step): the time one SIMD spends per slot."""
    import numpy as np
    import torch
    import w4a4_rank_corrected_smooth_amd as S
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S.device_check()
    stream = torch.cuda.current_stream(dev)
    grid, iters = 512, 60000
    sink = torch.zeros(grid, dtype=torch.int32, device=dev)
    peaks = {0: PEAK_FP6_TOPS, 1: PEAK_FP4_TOPS, 2: PEAK_BF16_TFLOPS, 3: PEAK_BF16_TFLOPS, 4: PEAK_INT8_TOPS}

    def timed(kind):
        for _ in range(3):
            S.measure_mfma(kind, iters, grid, sink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            S.measure_mfma(kind, iters, grid, sink)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    for kind, (label, ops) in S.MFMA_KINDS.items():
        t = timed(kind)
        n_instr = grid * 4 * 4 * iters
        rate = n_instr * ops / t / 1e12
        out = {"mfma": label, "grid": grid, "iters": iters, "ms": round(t * 1e3, 3),
               "rate_tops": round(rate, 1), "peak_tops": peaks[kind], "frac_of_peak": round(rate / peaks[kind], 4),
               "ns_per_instruction_per_simd": round(t * 1e9 * 1024 / n_instr, 2)}
        print(json.dumps(out), flush=True)
    # instruction mixes: time per slot (one chain step) on one SIMD
    for kind, label in S.MFMA_MIXES.items():
        t = timed(kind)
        n_slots = grid * 4 * 4 * iters
        print(json.dumps({"mix": label, "kind": kind, "grid": grid, "iters": iters, "ms": round(t * 1e3, 3),
                          "ns_per_slot_per_simd": round(t * 1e9 * 1024 / n_slots, 2)}), flush=True)


def hbm_floor(args):
    """The practical HBM rate at the bandwidth-bound kernels' own sizes and
    grids: a plain streaming read (and copy) of the quantiser's input (4608 x
    3072 and 4608 x 12288 bf16: 28.3 / 113.2 MB, grid (M/32) x splits) and
    of the W4A16 blob (18432 x 3072: 32 MB, grid N/16), each over rotating
    buffers whose total exceeds the 256 MB Infinity Cache, timed back to
    back; plus a sweep of grids.  One JSON line per case."""
    import torch
    import w4a4_rank_corrected_smooth_amd as S
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S.device_check()
    stream = torch.cuda.current_stream(dev)
    cases = [("k1_fc1_input", 4608 * 3072 * 2, 144 * 3), ("k1_fc2_input", 4608 * 12288 * 2, 144 * 3),
             ("k3_awq_blob", S._lib.awq_device_weights_bytes(18432, 3072), 18432 // 16)]
    for name, nbytes, kgrid in cases:
        nbytes = nbytes // 16 * 16
        RB = max(3, -(-640_000_000 // nbytes))
        src = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i) for i in range(RB)]
        dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        grids = sorted({kgrid, 256, 512, 1024, 2048, 4096, 8192})
        sink = torch.empty(max(grids), dtype=torch.int32, device=dev)
        res = {}
        for g in grids:
            us = back_to_back(lambda i: S.measure_stream(src[i % RB], g, sink=sink), stream)
            res[g] = round(nbytes / us / 1e3, 1)
        cus = back_to_back(lambda i: S.measure_stream(src[i % RB], kgrid, dst=dst), stream)
        best = max(res.values())
        print(json.dumps({"hbm_floor": name, "bytes": nbytes, "kernel_grid": kgrid, "rotating_sets": RB,
                          "read_gbs_by_grid": res, "read_gbs_at_kernel_grid": res[kgrid],
                          "read_gbs_best": best, "copy_gbs_at_kernel_grid": round(2 * nbytes / cus / 1e3, 1),
                          "read_frac_of_8tbs_best": round(best / PEAK_HBM_GBS, 4)}), flush=True)
        del src, dst
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU takes tens of milliseconds of sustained load to reach its
    # steady clocks; ~100 untimed steps (~70 ms) cover that
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sets", type=int, default=3, help="rotating copies of inputs and weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-unfused", action="store_true",
                    help="do not time the unfused pair (profiling runs: only the step's own kernels)")
    ap.add_argument("--skip-mx", action="store_true",
                    help="do not time the MXFP4 form of the MLP pair")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run an elementwise copy of known size (for HBM counter calibration)")
    ap.add_argument("--profiled-log", default=None,
                    help="with --summarize-profile: stdout of the traced bench run (its JSON line)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="CPU only: summarise rocprofv3 output into profiles/ and exit")
    ap.add_argument("--configs", action="store_true",
                    help="per-configuration kernel timings (one JSON line each) instead of the step")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="CPU only: summarise a rocprofv3 --pmc pass of the shader counters into profiles/")
    ap.add_argument("--summarize-counters-mem", metavar="PMC_DIR",
                    help="CPU only: summarise the second --pmc pass (waits, issue, LDS) into profiles/")
    ap.add_argument("--block", action="store_true",
                    help="launch study of one transformer block's calls, eager and as a HIP graph")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="CPU only: the oracle's forward timed per configuration (all threads; 1 thread for tiny and low-res)")
    ap.add_argument("--branch-ablation", action="store_true",
                    help="fused against unfused low-rank branch at QKV, fc1, fc2 and low-res (one JSON line)")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="achievable issue rate of each matrix instruction the path uses (registers only)")
    ap.add_argument("--hbm-floor", action="store_true",
                    help="streaming read/copy rates at the quantiser's and W4A16 kernel's sizes and grids")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "OUT_NAME", "TITLE", "COMMAND"),
                    help="CPU only: summarise a rocprofv3 trace (TRACE_DIR may be '-') into profiles/OUT_NAME")
    ap.add_argument("--summarize-mfma", metavar="JSONL",
                    help="CPU only: the --mfma-peak output as profiles/mfma_peak.md")
    ap.add_argument("--summarize-floor", nargs=2, metavar=("TRACE_DIR", "JSONL"),
                    help="CPU only: summarise a rocprofv3 trace of --hbm-floor into profiles/hbm_floor.md")
    ap.add_argument("--json", default=None, help="with --summarize-trace: the traced run's stdout")
    ap.add_argument("--note", default="", help="with --summarize-trace: a paragraph under the title")
    ap.add_argument("--summarize-configs", nargs=2, metavar=("TRACE_DIR", "SWEEP_JSONL"),
                    help="CPU only: summarise a rocprofv3 trace of --configs into profiles/ and exit")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, os.path.join(ROOT, "profiles", "mfma_peak.md"),
                       "python3 bench.py --mfma-peak")
        return
    if args.summarize_floor:
        t, j = args.summarize_floor
        summarize_floor(t, j, os.path.join(ROOT, "profiles", "hbm_floor.md"),
                        "rocprofv3 --kernel-trace --stats -f csv -d <dir> -- python3 bench.py --hbm-floor")
        return
    if args.summarize_trace:
        t, name, title, cmd = args.summarize_trace
        summarize_trace(None if t == "-" else t, os.path.join(ROOT, "profiles", name), title, cmd,
                        args.json, args.note)
        return
    if args.summarize_configs:
        t, j = args.summarize_configs
        summarize_configs(t, j, os.path.join(ROOT, "profiles", "kernels_all_configs.md"),
                          "rocprofv3 --kernel-trace --stats -f csv -d <dir> -- python3 bench.py --configs")
        return
    if args.summarize_counters_mem:
        base = "python3 bench.py --no-cpu-baseline --calibration-copy --skip-unfused --skip-mx"
        summarize_counters_mem(args.summarize_counters_mem,
                               os.path.join(ROOT, "profiles", "shader_counters_mem_flux_mlp_pair.md"),
                               f"rocprofv3 --pmc {' '.join(SQ_COUNTERS_MEM)} -f csv -d <dir> -- {base}")
        return
    if args.summarize_counters:
        base = "python3 bench.py --no-cpu-baseline --calibration-copy --skip-unfused --skip-mx"
        summarize_counters(args.summarize_counters, os.path.join(ROOT, "profiles", "shader_counters_flux_mlp_pair.md"),
                           f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} -f csv -d <dir> -- {base}")
        return
    if args.summarize_profile:
        t, fe, wr = args.summarize_profile
        base = "python3 bench.py --no-cpu-baseline --calibration-copy --skip-unfused --skip-mx"
        cmd = {"trace": f"rocprofv3 --kernel-trace --stats -f csv -d <dir> -- {base}",
               "fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -- {base}",
               "write": f"rocprofv3 --pmc WRITE_SIZE -f csv -d <dir> -- {base}"}
        summarize_profiles(t, fe, wr, os.path.join(ROOT, "profiles"), cmd, args.profiled_log)
        return
    if args.cpu_configs:
        cpu_configs(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library runs the layer on a single MI355X and "
              f"has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.configs:
        config_sweep(args)
        return
    if args.block:
        block_study(args)
        return
    if args.hbm_floor:
        hbm_floor(args)
        return
    if args.mfma_peak:
        mfma_peak(args)
        return
    if args.branch_ablation:
        branch_ablation_mode(args)
        return

    import numpy as np
    import torch
    import synth
    import w4a4_rank_corrected_smooth_amd as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S.device_check()
    R = max(1, args.sets)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------------------------------------------------------- setup
    log("generating the MLP pair (seed 2) and preparing fc1 on the host")
    fc1, W2, b2 = synth.mlp_cases()
    M, K1, N1 = fc1.M, fc1.K, fc1.N
    K2, N2 = N1, K1
    t0 = time.perf_counter()
    hw1 = S.prepare_weights(fc1.W, fc1.calib_absmax(), fc1.bias, 32)
    prep1 = time.perf_counter() - t0
    L1 = [S.Linear(hw1, dev) for _ in range(R)]
    X = [dev_bf16(fc1.X) for _ in range(R)]
    ws1 = [L1[0].new_workspace(M) for _ in range(R)]
    Y1 = [torch.empty((M, N1), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    log("calibrating fc2 on the device's own GELU(fc1) output")
    S.linear_forward(L1[0], X[0], out=Y1[0], gelu=True, workspace=ws1[0])
    torch.cuda.synchronize()
    ax2 = S.calibration_absmax(Y1[0][:64].cpu().view(torch.int16).numpy().view(np.uint16))
    t0 = time.perf_counter()
    hw2 = S.prepare_weights(W2, ax2, b2, 32)
    prep2 = time.perf_counter() - t0
    L2 = [S.Linear(hw2, dev) for _ in range(R)]
    ws2 = [L2[0].new_workspace(M) for _ in range(R)]
    Y2 = [torch.empty((M, N2), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    log("AWQ modulation projection 18432 x 3072 (seed 4)")
    a = synth.awq_case()
    q, s, z = S.awq_quantize_weights(a.W)
    A = [S.AwqLinear(q, s, z, dev) for _ in range(R)]
    xm = [torch.from_numpy(np.ascontiguousarray(a.x[:1])).to(dev) for _ in range(R)]
    ym = [torch.empty((1, a.N), dtype=torch.float16, device=dev) for _ in range(R)]
    torch.cuda.synchronize()

    if args.calibration_copy:
        src = torch.randn(CALIBRATION_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream(dev)
    NEV = 5

    def step(i, ev=None, fused=True):
        k = i % R

        def mark(j):
            if ev:
                ev[j].record(stream)
        mark(0)
        if fused:
            # fc1's GEMM quantises fc2's input in its epilogue (no fc1 output)
            S.mlp_quantize(L1[k], L2[k], X[k], ws1[k], ws2[k])
            mark(1)
            S.mlp_gemm1(L1[k], L2[k], M, ws1[k], ws2[k], gelu=True)
            mark(2)
            S.mlp_gemm2(L2[k], M, Y2[k], ws2[k])
            mark(3)
        else:
            S.linear_quantize(L1[k], X[k], ws1[k])
            mark(1)
            S.linear_gemm(L1[k], M, Y1[k], ws1[k], gelu=True)
            mark(2)
            S.linear_quantize(L2[k], Y1[k], ws2[k])
            S.linear_gemm(L2[k], M, Y2[k], ws2[k])
            mark(3)
        S.awq_forward(A[k], xm[k], out=ym[k])
        mark(4)

    def wall_pass(fused=True, sample_clock=False):
        """K uninstrumented steps between two device synchronisations; the
        shader clock is read while they run."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, fused=fused)
        mhz = read_sclk_mhz() if sample_clock else None
        torch.cuda.synchronize()
        return time.perf_counter() - t0, mhz

    log(f"warmup {args.warmup} steps, then at least {SETTLE_S} s of sustained load (clock settle)")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    settle_steps = settle(lambda i: step(i), SETTLE_S)
    log(f"timing {args.steps} steps (headline), then the same steps with per-kernel events")
    wall, sclk_mhz = wall_pass(True, sample_clock=True)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(NEV)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall_unfused = wall_fused2 = None
    if not args.skip_unfused:
        log(f"timing {args.steps} steps of the unfused pair, then the fused pair again")
        settle(lambda i: step(i, fused=False), 0.05)
        wall_unfused, _ = wall_pass(False)
        wall_fused2, _ = wall_pass(True)

    # bandwidth-bound kernels: back-to-back launches (no event between them)
    # over enough rotating buffers that a series exceeds the 256 MB
    # Infinity Cache
    k1_us = k3_us = None
    if not args.skip_unfused:
        log("K1 and K3 back to back over rotating buffers")
        RB = 10
        Xb = [X[i % R] if i < R else X[0].clone() for i in range(RB)]
        wsb = [ws1[i % R] if i < R else L1[0].new_workspace(M) for i in range(RB)]
        k1_us = back_to_back(lambda i: S.linear_quantize(L1[0], Xb[i % RB], wsb[i % RB]), stream)
        Ab = [A[i % R] if i < R else S.AwqLinear(q, s, z, dev) for i in range(RB)]
        k3_us = back_to_back(lambda i: S.awq_forward(Ab[i % RB], xm[0], out=ym[0]), stream)
        del Xb, wsb, Ab
        torch.cuda.empty_cache()

    branch = None
    if not args.skip_unfused:
        log("branch fusion ablation: QKV, fc1, fc2, low-res r128 fused and unfused")
        qc, lc = synth.qkv_case(), synth.lowres_case()
        Lq = S.Linear(S.prepare_weights(qc.W, qc.calib_absmax(), qc.bias, 32), dev)
        Ll = S.Linear(S.prepare_weights(lc.W, lc.calib_absmax(), lc.bias, 128), dev)
        xq = [dev_bf16(qc.X) for _ in range(2)]
        xl = [dev_bf16(lc.X) for _ in range(2)]
        S.linear_forward(L1[0], X[0], out=Y1[0], gelu=True, workspace=ws1[0])
        branch = branch_fusion(S, dev, stream, [("qkv", Lq, xq, False), ("fc1_gelu", L1[0], X[:2], True),
                                                ("fc2", L2[0], [Y1[0], Y1[0].clone()], False),
                                                ("lowres_r128", Ll, xl, False)])
        del Lq, Ll, xq, xl
        torch.cuda.empty_cache()

    mx = None
    if not args.skip_mx:
        mx = mx_pair(args, S, fc1, W2, b2, ax2, X, R, dev, stream)

    log("the GEMM's per-tile instruction mix, timed alone")
    step_ns = measure_step_ns(S, dev, stream)

    names = ["fc1_quantize", "fc1_gemm_gelu_quantize_fc2", "fc2_gemm", "awq_m1"]
    dur = {n: [] for n in names}
    span = []
    for ev in events:
        for j, n in enumerate(names):
            dur[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)   # us
        span.append(ev[0].elapsed_time(ev[NEV - 1]) * 1e3)
    avg = {n: float(np.mean(v)) for n, v in dur.items()}
    ms_per_step = wall / args.steps * 1e3
    ops_layer = 2.0 * M * N1 * K1            # = 2 * M * N2 * K2
    value = 2 * ops_layer / (ms_per_step * 1e-3) / 1e12

    k2_us = 0.5 * (avg["fc1_gemm_gelu_quantize_fc2"] + avg["fc2_gemm"])
    mix_us = 0.5 * (k2_mix_ceiling_us(step_ns, M, N1, K1) + k2_mix_ceiling_us(step_ns, M, N2, K2))
    achieved = ops_layer / (k2_us * 1e-6) / 1e12
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "k2_traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tj = json.load(f)
        if tj.get("source_hash") == source_hash():
            traffic = tj.get("bytes_per_launch")
    r = 32
    k1_bytes_fc1 = M * K1 * 2 + K1 * 4 + K1 * r * 2 + M * K1 // 2 + M * (K1 // 64) * 4 + M * r * 4
    awq_bytes = a.N * a.K // 2 + a.N * (a.K // 64) * 4 + a.K * 2 + a.N * 2
    out = {
        "metric": "W4A4+low-rank linear TOPS at Flux MLP shape; % of MI355X int8 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": "flux_mlp_pair_4608x3072x12288_r32_gelu+awq_mod_1x3072x18432",
                   "tokens": M, "d_model": K1, "d_ff": N1, "rank": 32, "group": 64,
                   "awq_rows": 1, "rotation_sets": R},
        # The INT4 x INT4 group sums run on gfx950's block-scaled matrix
        # instruction with fp6 E2M3 operands (codes -7..7 exact), so the
        # instruction's own peak (fp6, 10.1 POP/s) is the roofline; the
        # metric's int8 peak (5.0 POP/s) is reported beside it.
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP6_TOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP6_TOPS, 4),
                     "traffic": traffic, "kernel": "k2_w4a4_gemm",
                     "instruction": "v_mfma_scale_f32_32x32x64_f8f6f4 (fp6 E2M3 operands)",
                     "frac_int8_peak": round(achieved / PEAK_INT8_TOPS, 4), "peak_int8": PEAK_INT8_TOPS,
                     "ops_per_launch": ops_layer, "avg_launch_us": round(k2_us, 2),
                     # the main loop's instruction mix alone (matrix and vector
                     # instructions barely overlap on a SIMD): mean over fc1 and fc2
                     "mix_step_ns": round(step_ns, 2),
                     "mix_ceiling_us": round(mix_us, 2),
                     "frac_of_mix_ceiling": round(mix_us / k2_us, 4)},
        "kernels_us": {n: round(v, 2) for n, v in avg.items()},
        "event_step_us": round(float(np.mean(span)), 2),
        "settle_steps": settle_steps,
        "sclk_mhz_during_timing": sclk_mhz,
        "k1_gbs": ({"fc1": round(k1_bytes_fc1 / k1_us / 1e3, 1), "us_back_to_back": round(k1_us, 2),
                    "frac_hbm": round(k1_bytes_fc1 / k1_us / 1e3 / PEAK_HBM_GBS, 4)} if k1_us else None),
        "awq_gbs": ({"m1": round(awq_bytes / k3_us / 1e3, 1), "us_back_to_back": round(k3_us, 2),
                     "frac_hbm": round(awq_bytes / k3_us / 1e3 / PEAK_HBM_GBS, 4)} if k3_us else None),
        "unfused_pair": (None if wall_unfused is None else
                         {"ms_per_step": round(wall_unfused / args.steps * 1e3, 4),
                          "value": round(2 * ops_layer / (wall_unfused / args.steps) / 1e12, 2),
                          "fused_again_ms_per_step": round(wall_fused2 / args.steps * 1e3, 4)}),
        "weights_mb": footprint(S, [("fc1", N1, K1, 32), ("fc2", N2, K2, 32)], a),
        "branch_fusion": branch,
        "mxfp4_pair": mx,
        "prepare_s": {"fc1": round(prep1, 2), "fc2": round(prep2, 2)},
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
