#!/usr/bin/env python3
"""Benchmark: blockwise ring attention on one MI355X.

One step = one ring_attn_fwd_share call on the largest single-GPU forward
workload: rank 7's share of a 1,048,576-token causal ring (bf16, H=4,
d=128, P=8): its 131072 resident queries against all eight kv blocks in
ring order, each next block staged on the second stream.  Inputs are
resident in HBM.  Prints ONE JSON line:
  value        causal-adjusted TFLOP/s of the whole call (4 d FLOPs per
               unmasked query/key pair per query head), timed with HIP events
               on the caller's stream and the library's own kernel timing off
  roofline     the fused step kernel in a separate pass: algorithmic FLOPs per
               launch / mean launch time (HIP events on the compute stream)
               vs the bf16 dense MFMA peak; traffic and mfma_busy from the
               committed counter summaries (null once the kernel changed)
  cpu_baseline the fp64 oracle on a bounded row sample of the same workload
  prefill_32k  the causal contiguous ring B=1 H=32 N=32768 P=8 (whole call,
               roofline, cpu_baseline)
  striped_gqa  the causal striped GQA ring H=8/Hkv=2 N=131072 P=8 (same)
  decode       split-KV decode (16 sequences, H=32/Hkv=8, L=262144, d=128,
               P=8): algorithmic HBM GB/s, with its kernel's roofline
  backward     ring_attn_bwd on the 32k prefill workload: TFLOP/s at 10 d
               FLOPs per unmasked pair per query head
  backward_share  ring_attn_bwd_share on the headline workload (rank 7's
               share of the 1M-token ring), same FLOP count
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

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "causal ring-attn fwd TFLOP/s + % bf16 MFMA peak; split-KV decode HBM GB/s"

# The headline workload: the last rank's share of a 1,048,576-token ring (its
# q block against all eight kv blocks), the largest that fits one GPU.
SHARE = dict(B=1, H=4, Hkv=4, N=1048576, d=128, P=8, rank=7, layout="contiguous", causal=True, seed=4)
# The two other full-size forward workloads, measured beside it (same kernel,
# other shapes): the causal contiguous 32k prefill (whose backward the bench
# also times) and the striped GQA ring.
PREFILL = dict(B=1, H=32, Hkv=32, N=32768, d=128, P=8, layout="contiguous", causal=True, seed=2)
STRIPED = dict(B=1, H=8, Hkv=2, N=131072, d=128, P=8, layout="striped", causal=True, seed=3)
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


def measured_mfma_busy(key: str, source: str):
    """MFMA-busy fraction of the kernel on a workload from the committed
    counter summary (profiles/mfma.json), or None if its source changed."""
    try:
        rec = json.load(open(os.path.join(PROFILES, "mfma.json")))[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != source_sha(source):
        return None
    return {"busy": rec.get("mfma_busy"), "busy_rel_calibration_loop": rec.get("mfma_busy_rel_calibration"),
            "clock_ghz": rec.get("gui_clock_ghz")}


def host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}


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


def cpu_baseline(c, q, k, v, budget_s: float, share: bool) -> dict:
    """The fp64 oracle, as it is, on a seeded sample of query rows of the
    workload (two heads, uniformly random rows, each against all the keys
    it sees), timed on the host cores; FLOP/s at the same 4 d per pair."""
    import numpy as np
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(c["seed"])
    group = c["H"] // c["Hkv"]
    hs = sorted({0, c["H"] // 2})
    # local heads: query head i of the sample reads kv head i (its own group's)
    kv_of = [h // group for h in hs]
    qf = synth.as_f32(q[:, hs], "bf16")
    kf = synth.as_f32(k[:, kv_of], "bf16")
    vf = synth.as_f32(v[:, kv_of], "bf16")
    Nq = q.shape[2]
    q_pos = (oracle.host_positions(c["N"], c["P"], c["layout"])[c["rank"]] if share else np.arange(Nq))
    n_rows, elapsed, flops, rows_done = 16, 0.0, 0.0, 0
    while True:
        rows = np.sort(rng.integers(0, Nq, n_rows))
        t0 = time.perf_counter()
        oracle.attention(qf, kf, vf, causal=c["causal"], q_pos=q_pos, rows=rows,
                         heads=[(0, i) for i in range(len(hs))], threads=cores)
        dt = time.perf_counter() - t0
        elapsed += dt
        flops += 4.0 * c["d"] * float((q_pos[rows] + 1).sum()) * len(hs)
        rows_done += n_rows * len(hs)
        if elapsed >= budget_s:
            break
        n_rows = int(min(8192, max(n_rows * 2, n_rows * (budget_s - elapsed) / max(dt, 1e-3) * 0.5)))
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows_done} query rows (heads {hs}, uniformly random rows, each against every key it "
                      f"sees) of this workload, fp64, {elapsed:.1f} s", "seconds": elapsed, **host_cpu()}


def run_forward(args, c, share: bool, key: str, cpu_seconds: float) -> dict:
    """One full-size forward workload: whole calls timed with HIP events on
    the caller's stream (library kernel timing off), then a separate pass
    with the library's per-launch events for the step kernel's roofline."""
    import torch
    import blockwise_ring_attention_attn_amd as ra
    import synth
    B, H, Hkv, N, d, P = c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["P"]
    Nq = N // P if share else N
    q = synth.tensor(c["seed"], synth.TENSOR_Q, B, H, Nq, d, "bf16")
    k = synth.tensor(c["seed"], synth.TENSOR_K, B, Hkv, N, d, "bf16")
    v = synth.tensor(c["seed"], synth.TENSOR_V, B, Hkv, N, d, "bf16")
    qd, kd, vd = upload(q, "bf16"), upload(k, "bf16"), upload(v, "bf16")
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
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    # roofline pass: the library brackets each step-kernel launch with events
    n_prof = max(2, min(args.steps, int(2000.0 / max(ms, 1e-3))))
    ra.prof_enable(True)
    ra.prof_reset()
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    prof = ra.prof_read()
    ra.prof_enable(False)
    launches = prof["step_launches"]
    achieved = prof["step_flops"] / (prof["step_ms"] * 1e-3) / 1e12 if prof["step_ms"] > 0 else 0.0
    del qd, kd, vd, out, lse, ws
    torch.cuda.empty_cache()
    if share:
        what = (f"rank {c['rank']}'s share of a P={P} causal {c['layout']} ring over N={N} tokens: its {Nq} "
                f"queries against all {N} keys in ring order, bf16 B={B} H={H}/Hkv={Hkv} d={d}")
    else:
        what = f"causal {c['layout']} ring: bf16 B={B} H={H}/Hkv={Hkv} N={N} d={d}, P={P} virtual hosts"
    res = {
        "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "ms_per_step": ms, "steps": args.steps,
        "wall_s": wall, "flops_per_step": flops,
        "pct_bf16_mfma_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(f"step_bf16_kernel<128>:{key}", "attn_step.hip")
                     if key != "prefill_32k" else measured_traffic("step_bf16_kernel<128>", "attn_step.hip"),
                     "mfma_busy": measured_mfma_busy(f"step_bf16_kernel<128>:{key}", "attn_step.hip"),
                     "kernel": "step_bf16_kernel<128>", "launches_per_step": launches / n_prof,
                     "mean_launch_ms": prof["step_ms"] / max(1, launches),
                     "flops_per_launch": prof["step_flops"] / max(1, launches), "timed_calls": n_prof},
        "config": {"workload": what, **c},
    }
    if not args.no_cpu_baseline and cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(c, q, k, v, cpu_seconds, share)
    return res


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
            "mfma_busy": {k: measured_mfma_busy(f"{k}<128>:backward_prefill_32k", "attn_bwd.hip")
                          for k in ("bwd_dkdv_kernel", "bwd_dq_kernel")},
            "config": {"workload": "backward of the prefill workload (same shapes, upstream gradient seeded)"}}


def run_backward_share(args) -> dict:
    """ring_attn_bwd_share on the headline workload: rank 7's query block
    (after its forward share) against all 1,048,576 keys."""
    import torch
    import blockwise_ring_attention_attn_amd as ra
    import synth
    c = SHARE
    B, H, Hkv, N, d, P = c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["P"]
    Bl = N // P
    qd = upload(synth.tensor(c["seed"], synth.TENSOR_Q, B, H, Bl, d, "bf16"), "bf16")
    kd = upload(synth.tensor(c["seed"], synth.TENSOR_K, B, Hkv, N, d, "bf16"), "bf16")
    vd = upload(synth.tensor(c["seed"], synth.TENSOR_V, B, Hkv, N, d, "bf16"), "bf16")
    dod = upload(synth.tensor(c["seed"], synth.TENSOR_DOUT, B, H, Bl, d, "bf16"), "bf16")
    stream = torch.cuda.current_stream()
    kw = dict(P=P, rank=c["rank"], causal=c["causal"], layout=c["layout"], stream=stream)
    out, lse = ra.ring_attn_fwd_share(qd, kd, vd, **kw)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    nb = ra.load().ring_attn_bwd_share_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")

    def step():
        ra.ring_attn_bwd_share(qd, kd, vd, out, dod, lse, dq=dq, dk=dk, dv=dv, ws=ws, **kw)

    step()
    torch.cuda.synchronize()
    n = max(2, args.steps // 8)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(n):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / n
    flops = 2.5 * share_flops(c)
    tflops = flops / (ms * 1e-3) / 1e12
    del qd, kd, vd, dod, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"metric": "causal ring-attn bwd TFLOP/s (10 d per unmasked pair)", "value": tflops, "unit": "TFLOP/s",
            "ms_per_step": ms, "steps": n, "flops_per_step": flops,
            "pct_bf16_mfma_peak": 100.0 * tflops / MFMA_BF16_PEAK_TFLOPS,
            "mfma_busy": {k: measured_mfma_busy(f"{k}<128>:backward_share_1m", "attn_bwd.hip")
                          for k in ("bwd_dkdv_kernel", "bwd_dq_kernel")},
            "config": {"workload": "backward of rank 7's share of the 1,048,576-token ring (ring_attn_bwd_share; "
                                   "same shapes as the headline, upstream gradient seeded)"}}


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


def run_staging_cost(args) -> dict:
    """What the staging copies cost the step kernels that run beside them:
    the same forward calls with the ring exchange on (each step's kv blocks
    copied into staging buffers on the second stream while the previous step
    computes) and off (every block read in place, no copies), interleaved;
    whole-call time and the step kernels' mean launch time (HIP events on the
    compute stream)."""
    import torch
    import blockwise_ring_attention_attn_amd as ra
    import synth
    out = {}
    for key, c, share in (("prefill_32k", PREFILL, False), ("share_1m", SHARE, True)):
        B, H, Hkv, N, d, P = c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["P"]
        Nq = N // P if share else N
        qd = upload(synth.tensor(c["seed"], synth.TENSOR_Q, B, H, Nq, d, "bf16"), "bf16")
        kd = upload(synth.tensor(c["seed"], synth.TENSOR_K, B, Hkv, N, d, "bf16"), "bf16")
        vd = upload(synth.tensor(c["seed"], synth.TENSOR_V, B, Hkv, N, d, "bf16"), "bf16")
        o = torch.empty_like(qd)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda:0")
        stream = torch.cuda.current_stream()

        def step():
            if share:
                ra.ring_attn_fwd_share(qd, kd, vd, P=P, rank=c["rank"], causal=True, layout=c["layout"], out=o,
                                       lse=lse, stream=stream)
            else:
                ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=c["layout"], out=o, lse=lse, stream=stream)

        step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        n = max(2, min(20, int(1.0 / max(time.perf_counter() - t0, 1e-3))))
        res = {"on": [], "off": []}
        try:
            for rnd in range(6):
                for mode in (("on", "off") if rnd % 2 == 0 else ("off", "on")):
                    ra.debug_set_staging(mode == "on")
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
                    res[mode].append((ev0.elapsed_time(ev1) / n, prof["step_ms"] / max(1, prof["step_launches"])))
        finally:
            ra.debug_set_staging(True)
            ra.prof_enable(False)
        med = lambda xs: sorted(xs)[len(xs) // 2]
        on_call, off_call = med([x for x, _ in res["on"]]), med([x for x, _ in res["off"]])
        on_k, off_k = med([y for _, y in res["on"]]), med([y for _, y in res["off"]])
        out[key] = {"call_ms_staged": on_call, "call_ms_in_place": off_call,
                    "step_kernel_ms_staged": on_k, "step_kernel_ms_in_place": off_k,
                    "step_kernel_slowdown_pct": 100.0 * (on_k / off_k - 1.0),
                    "call_slowdown_pct": 100.0 * (on_call / off_call - 1.0), "calls_per_sample": n}
        del qd, kd, vd, o, lse
        torch.cuda.empty_cache()
    return out


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
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time on the headline workload")
    ap.add_argument("--cpu-seconds-other", type=float, default=6.0,
                    help="oracle time on each of the other two forward workloads")
    ap.add_argument("--no-other-forward", action="store_true",
                    help="skip the 32k prefill and striped GQA forward workloads")
    ap.add_argument("--calib-iters", type=int, default=8192)
    ap.add_argument("--only", choices=("prefill", "decode", "backward", "backward_share", "striped", "share",
                                       "mfma_calib", "staging_cost"),
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
    if args.only == "staging_cost":
        print(json.dumps(run_staging_cost(args)), flush=True)
        return
    if args.only == "decode":
        print(json.dumps(run_decode(args)), flush=True)
        return
    if args.only == "backward":
        print(json.dumps(run_backward(args)), flush=True)
        return
    if args.only == "backward_share":
        print(json.dumps(run_backward_share(args)), flush=True)
        return
    if args.only in ("striped", "share", "prefill"):
        c, share = {"striped": (STRIPED, False), "share": (SHARE, True), "prefill": (PREFILL, False)}[args.only]
        key = {"striped": "striped_gqa", "share": "share_1m", "prefill": "prefill_32k"}[args.only]
        print(json.dumps(run_forward(args, c, share, key, 0.0 if args.no_cpu_baseline else args.cpu_seconds)),
              flush=True)
        return
    head = run_forward(args, SHARE, True, "share_1m", args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {**head["config"], "global_batch": SHARE["B"], "seq_len": SHARE["N"],
                   "parallelism": "1 GPU: one device's share of a P=8 ring (the other 7 hosts' kv blocks staged "
                                  "on a second stream)"},
        "pct_bf16_mfma_peak": head["pct_bf16_mfma_peak"],
        "algorithmic_flops_per_step": head["flops_per_step"],
        "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if not args.no_other_forward:
        line["prefill_32k"] = run_forward(args, PREFILL, False, "prefill_32k", args.cpu_seconds_other)
        line["striped_gqa"] = run_forward(args, STRIPED, False, "striped_gqa", args.cpu_seconds_other)
    if not args.no_decode:
        line["decode"] = run_decode(args)
    if not args.no_backward:
        line["backward"] = run_backward(args)
        line["backward_share"] = run_backward_share(args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
