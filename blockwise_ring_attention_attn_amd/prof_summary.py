"""Turn rocprofv3 outputs into the short text summaries kept in profiles/.

    python -m blockwise_ring_attention_attn_amd.prof_summary stats <out_dir> <summary.md> "<command>"
        kernel-trace statistics (the *_kernel_stats.csv of --stats)
    python -m blockwise_ring_attention_attn_amd.prof_summary traffic <fetch_dir> <write_dir> <calib_mib> \\
        <kernel_substring> <kernel_key> <source_file> <summary.md> "<command>"
        FETCH_SIZE / WRITE_SIZE per dispatch (KiB), each scaled by what the
        same counter reads for the plain calibration copy of <calib_mib> MiB;
        writes profiles/traffic.json[<kernel_key>] with bytes per launch and
        the sha256 of the kernel's source file.
    python -m blockwise_ring_attention_attn_amd.prof_summary overlap <out_dir> <summary.md> "<command>"
        from the kernel trace of the bench command: over the forward calls of
        the prefill workload (the step kernels before the first decode
        kernel), the compute stream's idle share and how much of the staging
        copies' time runs under a step kernel.
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


def overlap(out_dir: str, summary: str, command: str) -> None:
    rows = list(csv.DictReader(open(_one(os.path.join(out_dir, "**", "*_kernel_trace.csv")))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    t_end = min((int(r["Start_Timestamp"]) for r in rows if "decode_partial_kernel" in r["Kernel_Name"]),
                default=None)
    if t_end is None:
        raise SystemExit("no decode kernel in the trace: cannot delimit the prefill calls")
    steps = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
             if "step_bf16_kernel" in r["Kernel_Name"] and int(r["End_Timestamp"]) <= t_end]
    if not steps:
        raise SystemExit("no step kernel before the first decode kernel")
    w0, w1 = steps[0][0], max(b for _, b in steps)
    busy = _union(steps)
    busy_ns = sum(b - a for a, b in busy)
    copies = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
              if "copyBuffer" in r["Kernel_Name"] and w0 <= int(r["Start_Timestamp"]) < w1]
    copy_ns = sum(b - a for a, b in copies)
    under = sum(_covered(a, b, busy) for a, b in copies)
    lines = [f"# Ring overlap ({os.path.basename(summary)})", "", "Command:", "", "```", command, "```", "",
             "Window: from the first step kernel to the last one that ends before the first decode kernel "
             "(the forward calls of the prefill workload, warm-up included).", "",
             "| Figure | Value |", "|---|---|",
             f"| step kernels | {len(steps)} |",
             f"| window | {(w1 - w0) / 1e6:.3f} ms |",
             f"| compute stream busy (union of step kernels) | {busy_ns / 1e6:.3f} ms |",
             f"| compute stream idle | {100.0 * (1 - busy_ns / (w1 - w0)):.2f}% |",
             f"| staging copy kernels | {len(copies)}, {copy_ns / 1e6:.3f} ms |",
             f"| copy time under a step kernel | {100.0 * under / max(copy_ns, 1):.1f}% |", ""]
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
        overlap(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 5 and sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 10 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10])
    else:
        print(__doc__)
        sys.exit(2)
