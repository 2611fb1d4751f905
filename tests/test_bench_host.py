"""Host-side checks of bench.py's algorithmic FLOP counts (no GPU).

The bench divides closed-form pair counts by measured time; these tests
check the closed forms against the oracle's exact per-block counts of
unmasked (query, key) pairs, taken from the positions of each layout."""
import os
import sys

import oracle

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _exact(c, host=None):
    pc = oracle.pair_counts(c["N"], c["P"], c["layout"], c["causal"])
    pairs = int(pc.sum()) if host is None else int(pc[host].sum())
    return 4.0 * c["d"] * pairs * c["B"] * c["H"]


def test_prefill_flops_match_exact_pair_counts():
    assert bench.prefill_flops(bench.PREFILL) == _exact(bench.PREFILL)
    assert bench.prefill_flops(bench.STRIPED) == _exact(bench.STRIPED)


def test_share_flops_match_exact_pair_counts():
    c = bench.SHARE
    assert bench.share_flops(c) == _exact(c, host=c["rank"])
    small = dict(c, N=1024, rank=3)
    assert bench.share_flops(small) == _exact(small, host=3)


def test_decode_bytes_counts_kv_once():
    c = bench.DECODE
    kv = 2 * c["B"] * c["Hkv"] * c["L"] * c["d"] * 2
    assert kv <= bench.decode_bytes(c) <= kv * 1.001


def test_overlap_summary_on_a_synthetic_trace(tmp_path):
    """Idle share and copy overlap from a hand-made kernel trace: step kernels
    [0,10) and [12,20) ns, copies [5,15) and [30,31) (the latter after the
    window), then a decode kernel at 40."""
    from blockwise_ring_attention_attn_amd import prof_summary
    d = tmp_path / "t"
    d.mkdir()
    rows = [("step_bf16_kernel<128>", 0, 10), ("__amd_rocclr_copyBuffer", 5, 15),
            ("step_bf16_kernel<128>", 12, 20), ("__amd_rocclr_copyBuffer", 30, 31),
            ("decode_partial_kernel<128>", 40, 50)]
    with open(d / "x_kernel_trace.csv", "w") as f:
        f.write('"Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for n, a, b in rows:
            f.write(f'"{n}",{a},{b}\n')
    out = tmp_path / "s.md"
    prof_summary.overlap(str(d), str(out), "cmd")
    text = out.read_text()
    assert "| compute kernels | 2 |" in text
    assert "| compute stream idle | 10.00% |" in text          # 2 of 20 ns
    assert "| staging copy kernels | 1," in text               # the copy at 30 is outside the window
    assert "| copy time under a compute kernel | 80.0% |" in text  # [5,10) and [12,15) of [5,15)


def test_overlap_summary_of_other_compute_kernels(tmp_path):
    """Without a decode kernel the window spans every listed compute kernel
    (here the two backward kernels)."""
    from blockwise_ring_attention_attn_amd import prof_summary
    d = tmp_path / "t"
    d.mkdir()
    rows = [("bwd_dkdv_kernel<128, 0>", 0, 10), ("bwd_dq_kernel<128, 0>", 10, 16), ("__amd_rocclr_copyBuffer", 2, 6),
            ("bwd_dkdv_kernel<128, 0>", 20, 40)]
    with open(d / "x_kernel_trace.csv", "w") as f:
        f.write('"Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for n, a, b in rows:
            f.write(f'"{n}",{a},{b}\n')
    out = tmp_path / "s.md"
    prof_summary.overlap(str(d), str(out), "cmd", "bwd_dkdv_kernel,bwd_dq_kernel")
    text = out.read_text()
    assert "| compute kernels | 3 |" in text
    assert "| compute stream idle | 10.00% |" in text          # [16,20) of [0,40)
    assert "| copy time under a compute kernel | 100.0% |" in text


def test_cpu_baseline_runs_the_oracle_on_each_workload_shape():
    """The CPU baseline leg on tiny versions of the three forward workloads
    (the share with its rank's positions, GQA heads mapped to their kv head)."""
    import synth
    for c, share in ((dict(bench.SHARE, N=1024, H=4, Hkv=4), True), (dict(bench.STRIPED, N=512), False),
                     (dict(bench.PREFILL, N=256, H=4, Hkv=4), False)):
        Nq = c["N"] // c["P"] if share else c["N"]
        q = synth.tensor(c["seed"], synth.TENSOR_Q, c["B"], c["H"], Nq, c["d"], "bf16")
        k = synth.tensor(c["seed"], synth.TENSOR_K, c["B"], c["Hkv"], c["N"], c["d"], "bf16")
        v = synth.tensor(c["seed"], synth.TENSOR_V, c["B"], c["Hkv"], c["N"], c["d"], "bf16")
        r = bench.cpu_baseline(c, q, k, v, 0.05, share)
        assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1
        assert r["os_cpu_count"] >= 1 and r["cpu_model"]
