#!/usr/bin/env python3
"""Benchmark: blockwise ring attention on one MI355X.

One step = one ring_attn_fwd call over the whole causal prefill workload
(bf16, B=1, H=32, N=32768, d=128, contiguous layout, P=8 virtual hosts,
all ring steps with the staging copies on the second stream), inputs already
resident in HBM.  Prints ONE JSON line:
  value        causal-adjusted TFLOP/s of the whole call (4 d FLOPs per
               unmasked query/key pair per query head)
  roofline     the fused step kernel: algorithmic FLOPs per launch / mean
               launch time (HIP events on the compute stream) vs the bf16
               dense MFMA peak
  cpu_baseline the fp64 oracle on a bounded row sample of the same workload
  decode       split-KV decode (16 sequences, H=32/Hkv=8, L=262144, d=128,
               P=8): algorithmic HBM GB/s, with its kernel's roofline
  backward     ring_attn_bwd on the prefill workload (reverse ring,
               recomputation): TFLOP/s at 10 d FLOPs per unmasked pair per
               query head (the five products QK^T, dO V^T, P^T dO, dS K,
               dS^T Q)
  striped_gqa  the striped GQA ring (bf16 H=8/Hkv=2, N=131072, P=8):
               TFLOP/s of the whole call
  share_1m     rank 7's share of a 1,048,576-token causal ring (bf16 H=4):
               TFLOP/s of the whole call
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "causal ring-attn fwd TFLOP/s + % bf16 MFMA peak; split-KV decode HBM GB/s"

PREFILL = dict(B=1, H=32, Hkv=32, N=32768, d=128, P=8, layout="contiguous", causal=True, seed=2)
# The two other full-size forward workloads, measured beside the headline one
# (same kernel, other shapes): the striped GQA ring, and the last rank's share
# of a 1,048,576-token ring (its q block against all eight kv blocks).
STRIPED = dict(B=1, H=8, Hkv=2, N=131072, d=128, P=8, layout="striped", causal=True, seed=3)
SHARE = dict(B=1, H=4, Hkv=4, N=1048576, d=128, P=8, rank=7, layout="contiguous", causal=True, seed=4)
DECODE = dict(B=16, H=32, Hkv=8, L=262144, d=128, P=8, seed=5)


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "blockwise_ring_attention_attn_amd", "csrc")


def source_sha(name: str) -> str:
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()


def measured_traffic(kernel: str, source: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/traffic.json), or None if the kernel source changed since."""
    try:
        rec = json.load(open(os.path.join(PROFILES, "traffic.json")))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_sha(source):
        return None
    return rec.get("bytes_per_launch")


def calibration_copy(mib: int) -> None:
    """A plain device-to-device copy of known size, for counter calibration."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def prefill_flops(c) -> float:
    N = c["N"]
    pairs = N * (N + 1) // 2 if c["causal"] else N * N
    return 4.0 * c["d"] * pairs * c["B"] * c["H"]


def share_flops(c) -> float:
    """Rank r's query block (positions r Bl + i) against all N keys, causal."""
    N, P, r = c["N"], c["P"], c["rank"]
    Bl = N // P
    pairs = r * Bl * Bl + Bl * (Bl + 1) // 2 if c["causal"] else Bl * N
    return 4.0 * c["d"] * pairs * c["B"] * c["H"]


def decode_bytes(c) -> float:
    B, H, Hkv, L, d, P = c["B"], c["H"], c["Hkv"], c["L"], c["d"], c["P"]
    kv = 2.0 * B * Hkv * L * d * 2          # K and V read once (GQA: not x H/Hkv)
    qo = 2.0 * B * H * d * 2 + B * H * 4    # q read, O (bf16) and lse written
    part = 2.0 * B * H * P * (d + 1) * 4    # per-ring-block fp32 partials written and read
    return kv + qo + part


def upload(x, dtype):
    import numpy as np
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(x).to("cuda:0")


def cpu_baseline(c, q, k, v, budget_s: float = 12.0) -> dict:
    """The fp64 oracle, as it is, on a seeded sample of query rows."""
    import numpy as np
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(c["seed"])
    heads = [(0, h) for h in (0, c["H"] // 2)]
    qf = synth.as_f32(q[:, :c["H"]], "bf16")
    kf = synth.as_f32(k, "bf16")
    vf = synth.as_f32(v, "bf16")
    n_rows = 64
    elapsed, flops, rows_done = 0.0, 0.0, 0
    while True:
        rows = np.sort(rng.integers(0, c["N"], n_rows))
        t0 = time.perf_counter()
        oracle.attention(qf, kf, vf, causal=True, rows=rows, heads=heads, threads=cores)
        dt = time.perf_counter() - t0
        elapsed += dt
        flops += 4.0 * c["d"] * float((rows + 1).sum()) * len(heads)
        rows_done += n_rows * len(heads)
        if elapsed >= budget_s:
            break
        n_rows = int(min(4096, max(n_rows * 2, n_rows * (budget_s - elapsed) / max(dt, 1e-3) * 0.5)))
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_done} query rows (heads 0 and {c['H'] // 2}, uniformly random positions, "
                      f"causal prefix of each row) of the prefill workload, fp64, {elapsed:.1f} s",
            "seconds": elapsed}


def run_prefill(args) -> dict:
    import torch
    import blockwise_ring_attention_attn_amd as ra
    import synth
    c = PREFILL
    q, k, v = synth.qkv(c["seed"], c["B"], c["H"], c["Hkv"], c["N"], c["d"], "bf16")
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
    out = torch.empty_like(qd)
    lse = torch.empty((c["B"], c["H"], c["N"]), dtype=torch.float32, device="cuda:0")
    nb = ra.ring_attn_fwd_ws_bytes(c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["P"], ra.RA_BF16)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        ra.ring_attn_fwd(qd, kd, vd, P=c["P"], causal=c["causal"], layout=c["layout"], out=out, lse=lse,
                         ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ra.prof_enable(True)
    ra.prof_reset()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = ra.prof_read()
    ra.prof_enable(False)
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = prefill_flops(c)
    tflops = flops / (ms * 1e-3) / 1e12
    launches = prof["step_launches"]
    kern_ms = prof["step_ms"] / max(1, launches)
    achieved = prof["step_flops"] / (prof["step_ms"] * 1e-3) / 1e12 if prof["step_ms"] > 0 else 0.0
    res = {
        "value": tflops, "ms_per_step": ms, "wall_s": wall, "flops": flops,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic("step_bf16_kernel<128>", "attn_step.hip"),
                     "kernel": "step_bf16_kernel<128>", "launches_per_step": launches / args.steps,
                     "mean_launch_ms": kern_ms,
                     "flops_per_launch": prof["step_flops"] / max(1, launches)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(c, q, k, v, args.cpu_seconds)
    del qd, kd, vd, out, lse, ws
    torch.cuda.empty_cache()
    return res


def run_forward_other(args, c, share: bool) -> dict:
    """Throughput of one of the other full-size forward workloads (HIP events
    around whole calls on the caller's stream; step-kernel launches timed on
    the compute stream as for the headline workload)."""
    import torch
    import blockwise_ring_attention_attn_amd as ra
    import synth
    B, H, Hkv, N, d, P = c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["P"]
    Nq = N // P if share else N
    qd = upload(synth.tensor(c["seed"], synth.TENSOR_Q, B, H, Nq, d, "bf16"), "bf16")
    kd = upload(synth.tensor(c["seed"], synth.TENSOR_K, B, Hkv, N, d, "bf16"), "bf16")
    vd = upload(synth.tensor(c["seed"], synth.TENSOR_V, B, Hkv, N, d, "bf16"), "bf16")
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda:0")
    lib = ra.load()
    nb = (lib.ring_attn_fwd_share_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16) if share
          else ra.ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16))
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        if share:
            ra.ring_attn_fwd_share(qd, kd, vd, P=P, rank=c["rank"], causal=c["causal"], layout=c["layout"],
                                   out=out, lse=lse, ws=ws, stream=stream)
        else:
            ra.ring_attn_fwd(qd, kd, vd, P=P, causal=c["causal"], layout=c["layout"], out=out, lse=lse, ws=ws,
                             stream=stream)

    flops = share_flops(c) if share else prefill_flops(c)
    step()
    torch.cuda.synchronize()
    # about 2 s of timed calls
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    n = int(min(20, max(3, 2.0 / max(time.perf_counter() - t0, 1e-3))))
    ra.prof_enable(True)
    ra.prof_reset()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(n):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    prof = ra.prof_read()
    ra.prof_enable(False)
    ms = ev0.elapsed_time(ev1) / n
    tflops = flops / (ms * 1e-3) / 1e12
    kern = prof["step_flops"] / (prof["step_ms"] * 1e-3) / 1e12 if prof["step_ms"] > 0 else 0.0
    del qd, kd, vd, out, lse, ws
    torch.cuda.empty_cache()
    if share:
        what = (f"rank {c['rank']} of a P={P} causal ring over N={N}: q {Nq} tokens against all {N} keys, "
                f"bf16 H={H} d={d}")
    else:
        what = f"causal {c['layout']} ring: bf16 B={B} H={H}/Hkv={Hkv} N={N} d={d}, P={P} virtual hosts"
    return {"value": tflops, "unit": "TFLOP/s", "ms_per_step": ms, "steps": n, "flops_per_step": flops,
            "pct_bf16_mfma_peak": 100.0 * tflops / MFMA_BF16_PEAK_TFLOPS,
            "step_kernels": {"achieved": kern, "unit": "TFLOP/s", "frac": kern / MFMA_BF16_PEAK_TFLOPS,
                             "launches_per_step": prof["step_launches"] / n,
                             "ms_per_step": prof["step_ms"] / n},
            "config": {"workload": what, **c}}


def run_backward(args) -> dict:
    import torch
    import blockwise_ring_attention_attn_amd as ra
    import synth
    c = PREFILL
    q, k, v = synth.qkv(c["seed"], c["B"], c["H"], c["Hkv"], c["N"], c["d"], "bf16")
    do = synth.tensor(c["seed"], synth.TENSOR_DOUT, c["B"], c["H"], c["N"], c["d"], "bf16")
    qd, kd, vd, dod = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16"), upload(do, "bf16")
    del q, k, v, do
    stream = torch.cuda.current_stream()
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=c["P"], causal=c["causal"], layout=c["layout"], stream=stream)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    nb = ra.load().ring_attn_bwd_ws_bytes(c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["P"], ra.RA_BF16)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")

    def step():
        ra.ring_attn_bwd(qd, kd, vd, out, dod, lse, P=c["P"], causal=c["causal"], layout=c["layout"], dq=dq, dk=dk,
                         dv=dv, ws=ws, stream=stream)

    step()
    torch.cuda.synchronize()
    n = max(3, args.steps // 4)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(n):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / n
    flops = 2.5 * prefill_flops(c)
    tflops = flops / (ms * 1e-3) / 1e12
    del qd, kd, vd, dod, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"metric": "causal ring-attn bwd TFLOP/s (10 d per unmasked pair)", "value": tflops, "unit": "TFLOP/s",
            "ms_per_step": ms, "steps": n, "flops_per_step": flops,
            "pct_bf16_mfma_peak": 100.0 * tflops / MFMA_BF16_PEAK_TFLOPS,
            "config": {"workload": "backward of the prefill workload (same shapes, upstream gradient seeded)"}}


def run_decode(args) -> dict:
    import torch
    import blockwise_ring_attention_attn_amd as ra
    import synth
    c = DECODE
    q, k, v = synth.qkv(c["seed"], c["B"], c["H"], c["Hkv"], c["L"], c["d"], "bf16", Nq=1)
    qd = upload(q, "bf16")
    kd = upload(k, "bf16")
    del k
    vd = upload(v, "bf16")
    del v
    out = torch.empty_like(qd)
    lse = torch.empty((c["B"], c["H"]), dtype=torch.float32, device="cuda:0")
    nb = ra.load().ring_attn_decode_ws_bytes(c["B"], c["H"], c["Hkv"], c["L"], c["d"], c["P"])
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        ra.ring_attn_decode(qd, kd, vd, P=c["P"], out=out, lse=lse, ws=ws, stream=stream)

    for _ in range(max(2, args.warmup)):
        step()
    torch.cuda.synchronize()
    ra.prof_enable(True)
    ra.prof_reset()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(args.steps, 10)
    ev0.record(stream)
    for _ in range(n):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    prof = ra.prof_read()
    ra.prof_enable(False)
    ms = ev0.elapsed_time(ev1) / n
    nbytes = decode_bytes(c)
    gbs = nbytes / (ms * 1e-3) / 1e9
    kern_achieved = prof["decode_bytes"] / (prof["decode_ms"] * 1e-3) / 1e9 if prof["decode_ms"] > 0 else 0.0
    del qd, kd, vd, out, lse, ws
    torch.cuda.empty_cache()
    return {
        "metric": "split-KV decode HBM GB/s", "value": gbs, "unit": "GB/s", "ms_per_step": ms, "steps": n,
        "frac_hbm_peak": gbs / HBM_PEAK_GBS, "bytes": nbytes,
        "config": {"workload": "decode: 16 sequences x 1 query token, H=32 / Hkv=8, L=262144, d=128, "
                               "P=8 ring blocks, bf16", **c},
        "roofline": {"bound": "hbm", "achieved": kern_achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kern_achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("decode_partial_kernel<128>", "decode.hip"),
                     "kernel": "decode_partial_kernel<128>",
                     "mean_launch_ms": prof["decode_ms"] / max(1, prof["decode_launches"]),
                     "bytes_per_launch": prof["decode_bytes"] / max(1, prof["decode_launches"])},
    }


def run_mfma_calib(args) -> dict:
    """The library's register-only bf16 MFMA loop: MFMAs issued, duration and
    rate (the counter calibration run; its rate is the practical MFMA peak)."""
    import torch
    import blockwise_ring_attention_attn_amd as ra
    stream = torch.cuda.current_stream()
    wgs, iters = 2048, args.calib_iters
    ra.diag_mfma_loop(wgs, 16, stream)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    n = ra.diag_mfma_loop(wgs, iters, stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    tflops = n * 32768.0 / (ms * 1e-3) / 1e12
    return {"kernel": "mfma_loop_kernel", "workgroups": wgs, "iters": iters, "mfma_count": n,
            "flops": n * 32768.0, "ms": ms, "tflops": tflops, "frac_nominal": tflops / MFMA_BF16_PEAK_TFLOPS}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-other-forward", action="store_true",
                    help="skip the striped GQA and 1M-share forward workloads")
    ap.add_argument("--calib-iters", type=int, default=8192)
    ap.add_argument("--only", choices=("prefill", "decode", "backward", "striped", "share", "mfma_calib"),
                    default=None,
                    help="run one workload only (profiling runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first do a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the ring's P hosts are emulated on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy_mib:
        calibration_copy(args.calib_copy_mib)
    if args.only == "mfma_calib":
        print(json.dumps(run_mfma_calib(args)), flush=True)
        return
    if args.only == "decode":
        print(json.dumps(run_decode(args)), flush=True)
        return
    if args.only == "backward":
        print(json.dumps(run_backward(args)), flush=True)
        return
    if args.only in ("striped", "share"):
        share = args.only == "share"
        print(json.dumps(run_forward_other(args, SHARE if share else STRIPED, share)), flush=True)
        return
    pre = run_prefill(args)
    c = PREFILL
    line = {
        "metric": METRIC,
        "value": pre["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill ring: bf16 B=1 H=32 N=32768 d=128, contiguous layout, "
                               "P=8 virtual hosts (all ring steps, KV staging on a second stream)",
                   "global_batch": c["B"], "seq_len": c["N"], "parallelism": "1 GPU, P=8 virtual ring hosts",
                   **c},
        "pct_bf16_mfma_peak": 100.0 * pre["value"] / MFMA_BF16_PEAK_TFLOPS,
        "algorithmic_flops_per_step": pre["flops"],
        "roofline": pre["roofline"],
    }
    if "cpu_baseline" in pre:
        line["cpu_baseline"] = pre["cpu_baseline"]
    if not args.no_decode and args.only is None:
        line["decode"] = run_decode(args)
    if not args.no_backward and args.only is None:
        line["backward"] = run_backward(args)
    if not args.no_other_forward and args.only is None:
        line["striped_gqa"] = run_forward_other(args, STRIPED, False)
        line["share_1m"] = run_forward_other(args, SHARE, True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
