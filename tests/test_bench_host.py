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
