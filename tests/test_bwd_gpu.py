"""GPU parity of ring_attn_bwd (bf16) against the fp64 backward oracle.

The pages fix no tolerance for gradients, so each element is checked
against a bound derived from the arithmetic of the bf16 path (it is stated
with the design notes): the GPU rounds P and dS to bf16 (relative 2^-9) as
MFMA operands, forms delta = dO . O from the forward's bf16 output, uses
the forward's fp32 lse, and rounds dq, dk, dv to bf16.  With the oracle's
exact P, dS, D (on the same bf16 inputs) the first-order error of each
gradient entry is at most

    dV_jc:  e * sum_i P_ij |dO_ic|
    dK_jc:  scale * sum_i (e |dS_ij| + dD_ij) |q_ic|
    dQ_ic:  scale * sum_j (e |dS_ij| + dD_ij) |k_jc|
    dD_ij = P_ij * e * sum_c |dO_ic| (|O_ic| + sum_j' P_ij' |v_j'c|)

plus e |ref| for the output rounding, with e = 2^-8 (twice the bf16 unit
roundoff, covering the fp32 exp / lse / accumulation terms).  The test
asserts |got - ref| <= 2 * bound + 1e-6 everywhere.
"""
import math

import numpy as np
import pytest

import blockwise_ring_attention_attn_amd as ra
import oracle
import synth
from _util import from_dev, host_vals, to_dev

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -8


def _inputs(seed, B, H, Hkv, N, d):
    print(f"\n[bwd case] seed={seed} B={B} H={H}/{Hkv} N={N} d={d}", flush=True)
    q, k, v = synth.qkv(seed, B, H, Hkv, N, d, "bf16")
    do = synth.tensor(seed, synth.TENSOR_DOUT, B, H, N, d, "bf16")
    return q, k, v, do


def _bounds(qh, kh, vh, doh, parts, B, H, Hkv, scale, dq_ref, dk_ref, dv_ref):
    """Element-wise error bounds of the bf16 path (see the module docstring)."""
    group = H // Hkv
    bq = np.zeros_like(dq_ref)
    bk = np.zeros_like(dk_ref)
    bv = np.zeros_like(dv_ref)
    for (b, h), p in parts.items():
        g = h // group
        P, dS = p["P"], p["dS"]
        Q, K, V, dO = (x.astype(np.float64) for x in (qh[b, h], kh[b, g], vh[b, g], doh[b, h]))
        O = P @ V
        o_err = np.abs(O) + P @ np.abs(V)                        # |O| + sum_j P |v|
        dD = P * (EPS * (np.abs(dO) * o_err).sum(axis=1))[:, None]
        w = EPS * np.abs(dS) + dD
        bq[b, h] = scale * (w @ np.abs(K))
        bk[b, g] += scale * (w.T @ np.abs(Q))
        bv[b, g] += EPS * (P.T @ np.abs(dO))
    bq += EPS * np.abs(dq_ref)
    bk += EPS * np.abs(dk_ref)
    bv += EPS * np.abs(dv_ref)
    return bq, bk, bv


def _run(seed, B, H, Hkv, N, d, P, causal, layout):
    import torch
    q, k, v, do = _inputs(seed, B, H, Hkv, N, d)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=causal, layout=layout)
    dq, dk, dv = ra.ring_attn_bwd(qd, kd, vd, out, dod, lse, P=P, causal=causal, layout=layout)
    torch.cuda.synchronize()
    return q, k, v, do, from_dev(dq), from_dev(dk), from_dev(dv)


def _check(seed, B, H, Hkv, N, d, P, causal, layout):
    q, k, v, do, dq, dk, dv = _run(seed, B, H, Hkv, N, d, P, causal, layout)
    qh, kh, vh, doh = (host_vals(x, "bf16") for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    dq_r, dk_r, dv_r, parts = oracle.attention_bwd(qh, kh, vh, doh, scale=scale, causal=causal, parts=True)
    bq, bk, bv = _bounds(qh, kh, vh, doh, parts, B, H, Hkv, scale, dq_r, dk_r, dv_r)
    what = f"bwd B={B} H={H}/{Hkv} N={N} d={d} P={P} causal={causal} {layout}"
    for name, got, ref, bnd in (("dq", dq, dq_r, bq), ("dk", dk, dk_r, bk), ("dv", dv, dv_r, bv)):
        assert np.all(np.isfinite(got)), f"{what}: non-finite {name}"
        err = np.abs(got - ref)
        ratio = float((err / (2 * bnd + 1e-6)).max())
        rel = float(err.max() / max(np.abs(ref).max(), 1e-30))
        print(f"  {name}: max|err|={err.max():.3e} rel={rel:.2e} worst err/bound={ratio:.3f}")
        assert ratio <= 1.0, f"{what}: {name} exceeds its bound (err/bound {ratio:.3f})"
    return dq, dk, dv


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_bwd_causal_gqa_layouts(layout):
    """GQA 2:1, d = 128, P = 8, blocks of 130 rows (ragged against every tile)."""
    _check(41, 1, 2, 1, 16 * 65, 128, 8, True, layout)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_noncausal(d):
    _check(42, 1, 2, 2, 4 * 100, d, 4, False, "contiguous")


@pytest.mark.parametrize("N,P,layout", [(24, 8, "contiguous"), (16, 8, "zigzag"), (300, 1, "contiguous"),
                                        (3 * 257, 3, "striped")])
def test_bwd_ragged_small(N, P, layout):
    _check(43, 1, 2, 1, N, 64, P, True, layout)


def test_bwd_batched():
    _check(44, 2, 4, 2, 512, 128, 4, True, "contiguous")


def test_bwd_layout_and_P_invariance():
    """The same inputs through different layouts and ring sizes agree
    within twice the bf16 rounding of the results."""
    outs = [_run(45, 1, 2, 2, 1024, 128, P, True, lay)[4:] for lay, P in
            (("contiguous", 8), ("striped", 8), ("zigzag", 4), ("contiguous", 1))]
    for got in outs[1:]:
        for a, b in zip(got, outs[0]):
            scale = np.abs(b).max()
            assert np.abs(a - b).max() <= 2e-2 * scale
