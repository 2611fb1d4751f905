"""Turn rocprofv3 outputs into the short text summaries kept in profiles/.

    python -m blockwise_ring_attention_attn_amd.prof_summary stats <out_dir> <summary.md> "<command>"
        kernel-trace statistics (the *_kernel_stats.csv of --stats)
    python -m blockwise_ring_attention_attn_amd.prof_summary traffic <fetch_dir> <write_dir> <calib_mib> \\
        <kernel_substring> <kernel_key> <source_file> <summary.md> "<command>"
        FETCH_SIZE / WRITE_SIZE per dispatch (KiB), each scaled by what the
        same counter reads for the plain calibration copy of <calib_mib> MiB;
        writes profiles/traffic.json[<kernel_key>] with bytes per launch and
        the sha256 of the kernel's source file.
    python -m blockwise_ring_attention_attn_amd.prof_summary overlap <out_dir> <summary.md> "<command>" \
        [<compute kernel substrings, comma-separated>]
        from the kernel trace of a bench command: over the window from the
        first to the last compute kernel (the step kernels by default; only
        those before the first decode kernel when the trace holds one), the
        compute stream's idle share and how much of the staging copies' time
        runs under a compute kernel.
    python -m blockwise_ring_attention_attn_amd.prof_summary mfma <calib_p1> <calib_p2> <summary.md> <key> \
        <kernel_substring> <source_file> "<command>" <run_p1> <run_p2>
        MFMA and issue counters of one kernel, per launch, next to what the
        same counters read for the register-only MFMA calibration loop
        (bench.py --only mfma_calib: a known MFMA count); writes
        profiles/mfma.json[<key>] with the kernel's MFMA-busy fraction.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "blockwise_ring_attention_attn_amd", "csrc")


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def stats(out_dir: str, summary: str, command: str) -> None:
    f = _one(os.path.join(out_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(f)))
    lines = [f"# Kernel statistics ({os.path.basename(summary)})", "", "Command:", "", "```", command, "```", "",
             "| Kernel | Calls | Total ms | Average us | Min us | Max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows[:12]:
        name = r.get("Name") or r.get("KernelName") or "?"
        if len(name) > 80:
            name = name[:77] + "..."
        lines.append("| {} | {} | {:.3f} | {:.1f} | {:.1f} | {:.1f} | {:.1f} |".format(
            name.replace("|", "/"), r["Calls"], float(r["TotalDurationNs"]) / 1e6,
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    open(summary, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_dispatch(d: str):
    f = _one(os.path.join(d, "**", "*counter_collection.csv"))
    out = []
    for r in csv.DictReader(open(f)):
        out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def _union(iv):
    out = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _covered(a, b, merged) -> int:
    return sum(max(0, min(b, y) - max(a, x)) for x, y in merged)


def overlap(out_dir: str, summary: str, command: str, compute: str = "step_bf16_kernel") -> None:
    subs = [c for c in compute.split(",") if c]
    rows = list(csv.DictReader(open(_one(os.path.join(out_dir, "**", "*_kernel_trace.csv")))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    t_end = min((int(r["Start_Timestamp"]) for r in rows if "decode_partial_kernel" in r["Kernel_Name"]),
                default=None)
    t_end = t_end if t_end is not None else max(int(r["End_Timestamp"]) for r in rows) + 1
    steps = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
             if any(c in r["Kernel_Name"] for c in subs) and int(r["End_Timestamp"]) <= t_end]
    if not steps:
        raise SystemExit(f"no compute kernel ({compute}) in the window")
    w0, w1 = steps[0][0], max(b for _, b in steps)
    busy = _union(steps)
    busy_ns = sum(b - a for a, b in busy)
    copies = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
              if "copyBuffer" in r["Kernel_Name"] and w0 <= int(r["Start_Timestamp"]) < w1]
    copy_ns = sum(b - a for a, b in copies)
    under = sum(_covered(a, b, busy) for a, b in copies)
    lines = [f"# Ring overlap ({os.path.basename(summary)})", "", "Command:", "", "```", command, "```", "",
             f"Window: from the first compute kernel ({', '.join(subs)}) to the last one (before the first decode "
             "kernel, if any); warm-up calls and the gaps between calls included.", "",
             "| Figure | Value |", "|---|---|",
             f"| compute kernels | {len(steps)} |",
             f"| window | {(w1 - w0) / 1e6:.3f} ms |",
             f"| compute stream busy (union of compute kernels) | {busy_ns / 1e6:.3f} ms |",
             f"| compute stream idle | {100.0 * (1 - busy_ns / (w1 - w0)):.2f}% |",
             f"| staging copy kernels | {len(copies)}, {copy_ns / 1e6:.3f} ms |",
             f"| copy time under a compute kernel | {100.0 * under / max(copy_ns, 1):.1f}% |", ""]
    open(summary, "w").write("\n".join(lines))
    print("\n".join(lines))


def _counters(d: str, kernel_sub: str):
    """Per-dispatch counters of the kernels matching kernel_sub: a list of
    (duration_ns, {counter: value}); SQ counters summed over the instances
    the profiler reports, GRBM counters (one global value) taken as the max."""
    f = _one(os.path.join(d, "**", "*counter_collection.csv"))
    disp = {}
    for r in csv.DictReader(open(f)):
        if kernel_sub not in r["Kernel_Name"]:
            continue
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        ent = disp.setdefault(did, {"dur": 0.0, "c": {}})
        try:
            ent["dur"] = max(ent["dur"], float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
        except (KeyError, ValueError):
            pass
        name, val = r["Counter_Name"], float(r["Counter_Value"])
        if name.startswith("GRBM"):
            ent["c"][name] = max(ent["c"].get(name, 0.0), val)
        else:
            ent["c"][name] = ent["c"].get(name, 0.0) + val
    return [(e["dur"], e["c"]) for _, e in sorted(disp.items(), key=lambda kv: int(kv[0]))]


def _total(disp):
    tot = {}
    for _, c in disp:
        for k, v in c.items():
            tot[k] = tot.get(k, 0.0) + v
    return tot


def _gpu_agent(d: str):
    """(SIMD count, XCC count) of the GPU from the profiler's agent_info.csv."""
    for r in csv.DictReader(open(_one(os.path.join(d, "**", "*agent_info.csv")))):
        if r.get("Agent_Type", "").upper().endswith("GPU") or r.get("Name", "").startswith("gfx"):
            return int(r["Simd_Count"]), int(r["Num_Xcc"])
    raise SystemExit("no GPU agent in agent_info.csv")


def mfma(calib_p1, calib_p2, summary, key, kernel_sub, source, command, run_p1, run_p2) -> None:
    # The csv holds each counter summed over the instances the profiler
    # samples; GRBM_GUI_ACTIVE (busy cycles of the GPU) is counted once per
    # XCC, so the per-XCC value is the sum over the XCC count.
    SIMDS, n_xcc = _gpu_agent(run_p1)
    cal = _total(_counters(calib_p1, "mfma_loop_kernel")) | _total(_counters(calib_p2, "mfma_loop_kernel"))
    n_cal = len(_counters(calib_p1, "mfma_loop_kernel"))
    d1, d2 = _counters(run_p1, kernel_sub), _counters(run_p2, kernel_sub)
    if not d1 or not d2 or not n_cal:
        raise SystemExit("no matching dispatches")
    run = _total(d1) | _total(d2)
    cal["GRBM_GUI_ACTIVE"] /= n_xcc
    run["GRBM_GUI_ACTIVE"] /= n_xcc
    n = len(d1)
    cal_util = cal["SQ_VALU_MFMA_BUSY_CYCLES"] / (cal["GRBM_GUI_ACTIVE"] * SIMDS)
    util = run["SQ_VALU_MFMA_BUSY_CYCLES"] / (run["GRBM_GUI_ACTIVE"] * SIMDS)
    busy_per_mfma = cal["SQ_VALU_MFMA_BUSY_CYCLES"] / cal["SQ_INSTS_MFMA"]
    mops_per_mfma = cal["SQ_INSTS_VALU_MFMA_MOPS_BF16"] / cal["SQ_INSTS_MFMA"]
    dur_ns = sum(dd for dd, _ in d1)
    clock = run["GRBM_GUI_ACTIVE"] / dur_ns if dur_ns else float("nan")
    flops = run["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
    per = lambda name: run.get(name, float("nan")) / run["SQ_INSTS_MFMA"]
    rec = {"kernel": key, "launches": n, "mfma_busy": util, "mfma_busy_calibration": cal_util,
           "mfma_busy_rel_calibration": util / cal_util,
           "coexec_frac_of_busy": run["SQ_VALU_MFMA_COEXEC_CYCLES"] / run["SQ_VALU_MFMA_BUSY_CYCLES"],
           "executed_tflops_from_counters": flops / (dur_ns * 1e-9) / 1e12 if dur_ns else None,
           "gui_clock_ghz": clock, "valu_per_mfma": per("SQ_INSTS_VALU"), "trans_per_mfma": per("SQ_INSTS_VALU_TRANS_F32"),
           "lds_per_mfma": per("SQ_INSTS_LDS"), "source": source,
           "source_sha256": hashlib.sha256(open(os.path.join(CSRC, source), "rb").read()).hexdigest(),
           "command": command}
    tj = os.path.join(ROOT, "profiles", "mfma.json")
    data = json.load(open(tj)) if os.path.exists(tj) else {}
    data[key] = rec
    json.dump(data, open(tj, "w"), indent=1, sort_keys=True)
    act = lambda c, name: c.get(name, float("nan"))
    lines = [f"# MFMA and issue counters: {key}", "", "Command (one run per counter pass; rocprofv3 --pmc, csv):", "",
             "```", command, "```", "",
             "Calibration: bench.py --only mfma_calib (the library's register-only loop of bf16 "
             "v_mfma_f32_32x32x16_bf16, eight independent chains per wave, known MFMA count) in the same two passes.",
             "", "| Figure | Calibration loop | Kernel |", "|---|---|---|",
             f"| dispatches | {n_cal} | {n} |",
             f"| SQ_INSTS_MFMA | {cal['SQ_INSTS_MFMA']:.4g} | {run['SQ_INSTS_MFMA']:.4g} |",
             f"| MOPS_BF16 per MFMA (x512 FLOPs) | {mops_per_mfma:.2f} | {run['SQ_INSTS_VALU_MFMA_MOPS_BF16'] / run['SQ_INSTS_MFMA']:.2f} |",
             f"| MFMA busy cycles per MFMA | {busy_per_mfma:.2f} | {run['SQ_VALU_MFMA_BUSY_CYCLES'] / run['SQ_INSTS_MFMA']:.2f} |",
             f"| MFMA busy = BUSY / (GRBM_GUI_ACTIVE x {SIMDS} SIMDs) | {cal_util:.3f} | {util:.3f} |",
             f"| kernel busy relative to the calibration loop | 1 | {util / cal_util:.3f} |",
             f"| co-issue: COEXEC / BUSY | {cal['SQ_VALU_MFMA_COEXEC_CYCLES'] / cal['SQ_VALU_MFMA_BUSY_CYCLES']:.3f} | {rec['coexec_frac_of_busy']:.3f} |",
             f"| VALU instructions per MFMA | {act(cal, 'SQ_INSTS_VALU') / cal['SQ_INSTS_MFMA']:.2f} | {rec['valu_per_mfma']:.2f} |",
             f"| of which transcendental (fp32) | {act(cal, 'SQ_INSTS_VALU_TRANS_F32') / cal['SQ_INSTS_MFMA']:.2f} | {rec['trans_per_mfma']:.2f} |",
             f"| LDS instructions per MFMA | {act(cal, 'SQ_INSTS_LDS') / cal['SQ_INSTS_MFMA']:.2f} | {rec['lds_per_mfma']:.2f} |",
             f"| SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES | {act(cal, 'SQ_ACTIVE_INST_VALU') / act(cal, 'SQ_WAVE_CYCLES'):.3f} | {act(run, 'SQ_ACTIVE_INST_VALU') / act(run, 'SQ_WAVE_CYCLES'):.3f} |",
             f"| SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES | {act(cal, 'SQ_ACTIVE_INST_LDS') / act(cal, 'SQ_WAVE_CYCLES'):.3f} | {act(run, 'SQ_ACTIVE_INST_LDS') / act(run, 'SQ_WAVE_CYCLES'):.3f} |",
             f"| SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES | {act(cal, 'SQ_WAIT_INST_ANY') / act(cal, 'SQ_WAVE_CYCLES'):.3f} | {act(run, 'SQ_WAIT_INST_ANY') / act(run, 'SQ_WAVE_CYCLES'):.3f} |",
             f"| SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS | - | {act(run, 'SQ_LDS_BANK_CONFLICT') / act(run, 'SQ_ACTIVE_INST_LDS'):.3f} |",
             f"| GRBM_GUI_ACTIVE per XCC / duration (GHz) | {cal['GRBM_GUI_ACTIVE'] / sum(dd for dd, _ in _counters(calib_p1, 'mfma_loop_kernel')):.3f} | {clock:.3f} |",
             f"| executed bf16 TFLOP/s (MOPS x 512 / duration) | - | {rec['executed_tflops_from_counters']:.1f} |",
             "", f"Kernel source: {source} (sha256 {rec['source_sha256'][:16]}...)", ""]
    open(summary, "w").write("\n".join(lines))
    print("\n".join(lines))


def traffic(fetch_dir, write_dir, calib_mib, kernel_sub, key, source, summary, command) -> None:
    calib_kib = float(calib_mib) * 1024.0
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _per_dispatch(d)
        # the calibration copy is the first dispatch whose counter is within 4x of its size
        cal = [v for n, v in rows if "copy" in n.lower() or "elementwise" in n.lower()]
        cal = [v for v in cal if calib_kib / 4 <= v <= calib_kib * 4]
        if not cal:
            raise SystemExit(f"{name}: calibration copy not found")
        factor = calib_kib / cal[0]
        vals = [v for n, v in rows if kernel_sub in n]
        res[name] = {"factor": factor, "kib_raw": vals, "bytes_scaled": [v * factor * 1024.0 for v in vals]}
    n = min(len(res["FETCH_SIZE"]["bytes_scaled"]), len(res["WRITE_SIZE"]["bytes_scaled"]))
    tot = [res["FETCH_SIZE"]["bytes_scaled"][i] + res["WRITE_SIZE"]["bytes_scaled"][i] for i in range(n)]
    per_launch = sum(tot) / max(1, n)
    sha = hashlib.sha256(open(os.path.join(CSRC, source), "rb").read()).hexdigest()
    tj = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(tj)) if os.path.exists(tj) else {}
    data[key] = {"bytes_per_launch": per_launch, "launches": n, "source": source, "source_sha256": sha,
                 "fetch_factor": res["FETCH_SIZE"]["factor"], "write_factor": res["WRITE_SIZE"]["factor"],
                 "command": command}
    json.dump(data, open(tj, "w"), indent=1, sort_keys=True)
    lines = [f"# HBM traffic of {key}", "", "Command (run once with --pmc FETCH_SIZE, once with --pmc WRITE_SIZE):",
             "", "```", command, "```", "",
             f"Calibration: a plain {calib_mib} MiB device copy reads FETCH_SIZE x{res['FETCH_SIZE']['factor']:.3f}"
             f" and WRITE_SIZE x{res['WRITE_SIZE']['factor']:.3f} of its true size; both counters are scaled by"
             " these factors.", "",
             "| Dispatch | FETCH KiB (raw) | WRITE KiB (raw) | HBM bytes (scaled) |", "|---|---|---|---|"]
    for i in range(n):
        lines.append(f"| {i} | {res['FETCH_SIZE']['kib_raw'][i]:.0f} | {res['WRITE_SIZE']['kib_raw'][i]:.0f} |"
                     f" {tot[i]:.4g} |")
    lines += ["", f"Mean HBM bytes per launch: {per_launch:.4g}", f"Kernel source: {source} (sha256 {sha[:16]}...)"]
    open(summary, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "overlap":
        overlap(*sys.argv[2:6])
    elif len(sys.argv) >= 11 and sys.argv[1] == "mfma":
        mfma(*sys.argv[2:11])
    elif len(sys.argv) >= 5 and sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 10 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10])
    else:
        print(__doc__)
        sys.exit(2)
