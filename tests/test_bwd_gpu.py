"""GPU parity of ring_attn_bwd (bf16 and fp32) against the fp64 backward oracle.

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

The fp32 path rounds nothing to bf16: the same bound with e = 2^-12 covers
its fp32 dot products over d <= 128 terms (d u |s|), the forward's fp32 row
sum over N <= 1024 keys behind lse (N u) and the gradients' sums over
N <= 1024 terms (N u), u = 2^-24, with room to spare (2^-12 = 2.4e-4 against
their 1.7e-4); a stray bf16 rounding (2^-9) would exceed it.
"""
import math

import numpy as np
import pytest

import blockwise_ring_attention_attn_amd as ra
import oracle
import synth
from _util import from_dev, host_vals, to_dev

pytestmark = pytest.mark.gpu

EPS = {"bf16": 2.0 ** -8, "f32": 2.0 ** -12}
# The element-wise bounds add |dS| |k| over every visible key and loosen as
# the key count grows (the terms' rounding errors largely cancel), so each
# gradient is also held, as a whole, to a normwise relative error: about
# five times the rounding of the results (bf16 2^-9, fp32 2^-24 times the
# key count), far below the share of one kv block out of P.
NORMWISE = {"bf16": 1e-2, "f32": 1e-4}


def _normwise(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


def _inputs(seed, B, H, Hkv, N, d, dtype="bf16"):
    print(f"\n[bwd case] seed={seed} B={B} H={H}/{Hkv} N={N} d={d} {dtype}", flush=True)
    q, k, v = synth.qkv(seed, B, H, Hkv, N, d, dtype)
    do = synth.tensor(seed, synth.TENSOR_DOUT, B, H, N, d, dtype)
    return q, k, v, do


def _bounds(qh, kh, vh, doh, parts, B, H, Hkv, scale, dq_ref, dk_ref, dv_ref, EPS):
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


def _run(seed, B, H, Hkv, N, d, P, causal, layout, dtype="bf16"):
    import torch
    q, k, v, do = _inputs(seed, B, H, Hkv, N, d, dtype)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=causal, layout=layout)
    dq, dk, dv = ra.ring_attn_bwd(qd, kd, vd, out, dod, lse, P=P, causal=causal, layout=layout)
    torch.cuda.synchronize()
    return q, k, v, do, from_dev(dq), from_dev(dk), from_dev(dv)


def _check(seed, B, H, Hkv, N, d, P, causal, layout, dtype="bf16"):
    q, k, v, do, dq, dk, dv = _run(seed, B, H, Hkv, N, d, P, causal, layout, dtype)
    qh, kh, vh, doh = (host_vals(x, dtype) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    dq_r, dk_r, dv_r, parts = oracle.attention_bwd(qh, kh, vh, doh, scale=scale, causal=causal, parts=True)
    bq, bk, bv = _bounds(qh, kh, vh, doh, parts, B, H, Hkv, scale, dq_r, dk_r, dv_r, EPS[dtype])
    what = f"bwd B={B} H={H}/{Hkv} N={N} d={d} P={P} causal={causal} {layout} {dtype}"
    for name, got, ref, bnd in (("dq", dq, dq_r, bq), ("dk", dk, dk_r, bk), ("dv", dv, dv_r, bv)):
        assert np.all(np.isfinite(got)), f"{what}: non-finite {name}"
        err = np.abs(got - ref)
        ratio = float((err / (2 * bnd + 1e-6)).max())
        rel = float(err.max() / max(np.abs(ref).max(), 1e-30))
        nw = _normwise(got, ref)
        print(f"  {name}: max|err|={err.max():.3e} rel={rel:.2e} normwise={nw:.2e} worst err/bound={ratio:.3f}")
        assert ratio <= 1.0, f"{what}: {name} exceeds its bound (err/bound {ratio:.3f})"
        assert nw <= NORMWISE[dtype], f"{what}: {name} normwise relative error {nw:.2e}"
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


def test_bwd_fp32_single_head_noncausal_P4():
    """The fp32 workload's shape (one head, N=1024, d=64, non-causal, P=4
    ring blocks of 256) through the fp32 backward."""
    _check(46, 1, 1, 1, 1024, 64, 4, False, "contiguous", "f32")


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_bwd_fp32_causal_gqa_layouts(layout):
    """fp32, GQA 2:1, d = 128, P = 8, blocks of 66 rows."""
    _check(47, 1, 4, 2, 16 * 33, 128, 8, True, layout, "f32")


def test_bwd_fp32_batched_ragged():
    _check(48, 2, 2, 1, 3 * 101, 64, 3, True, "striped", "f32")


# ---------------------------------------------------------------------------
# One device's share of the backward: host `rank`'s query rows against the
# whole sequence; the oracle is the plain backward of those rows (their
# global positions) against every key, whose dk, dv are exactly that rank's
# contribution.
# ---------------------------------------------------------------------------
def _share_inputs(seed, B, H, Hkv, N, d, P, rank, layout, dtype):
    q, k, v, do = _inputs(seed, B, H, Hkv, N, d, dtype)
    pos = oracle.host_positions(N, P, layout)[rank]
    qb = np.ascontiguousarray(q[:, :, pos])
    dob = np.ascontiguousarray(do[:, :, pos])
    return qb, k, v, dob, pos


def _run_share(qb, k, v, dob, P, rank, causal, layout, dtype):
    import torch
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (qb, k, v, dob))
    out, lse = ra.ring_attn_fwd_share(qd, kd, vd, P=P, rank=rank, causal=causal, layout=layout)
    dq, dk, dv = ra.ring_attn_bwd_share(qd, kd, vd, out, dod, lse, P=P, rank=rank, causal=causal, layout=layout)
    torch.cuda.synchronize()
    return from_dev(dq), from_dev(dk), from_dev(dv)


def _check_share(seed, B, H, Hkv, N, d, P, rank, causal, layout, dtype="bf16"):
    print(f"  share rank={rank} P={P} causal={causal} {layout}", flush=True)
    qb, k, v, dob, pos = _share_inputs(seed, B, H, Hkv, N, d, P, rank, layout, dtype)
    dq, dk, dv = _run_share(qb, k, v, dob, P, rank, causal, layout, dtype)
    qh, kh, vh, doh = (host_vals(x, dtype) for x in (qb, k, v, dob))
    scale = 1.0 / math.sqrt(d)
    dq_r, dk_r, dv_r, parts = oracle.attention_bwd(qh, kh, vh, doh, scale=scale, causal=causal, q_pos=pos,
                                                   parts=True)
    bq, bk, bv = _bounds(qh, kh, vh, doh, parts, B, H, Hkv, scale, dq_r, dk_r, dv_r, EPS[dtype])
    what = f"bwd_share B={B} H={H}/{Hkv} N={N} d={d} P={P} rank={rank} causal={causal} {layout} {dtype}"
    for name, got, ref, bnd in (("dq", dq, dq_r, bq), ("dk", dk, dk_r, bk), ("dv", dv, dv_r, bv)):
        assert np.all(np.isfinite(got)), f"{what}: non-finite {name}"
        err = np.abs(got - ref)
        ratio = float((err / (2 * bnd + 1e-6)).max())
        nw = _normwise(got, ref)
        print(f"  {name}: max|err|={err.max():.3e} normwise={nw:.2e} worst err/bound={ratio:.3f}")
        assert ratio <= 1.0, f"{what}: {name} exceeds its bound (err/bound {ratio:.3f})"
        assert nw <= NORMWISE[dtype], f"{what}: {name} normwise relative error {nw:.2e}"
    if causal:
        # keys after the rank's last query get exactly zero
        late = np.arange(N) > pos.max()
        assert not dk[:, :, late].any() and not dv[:, :, late].any()
    return dq, dk, dv


@pytest.mark.parametrize("layout,rank", [("contiguous", 0), ("contiguous", 7), ("contiguous", 3),
                                         ("striped", 5), ("zigzag", 2)])
def test_bwd_share_causal_gqa(layout, rank):
    """GQA 2:1, d = 128, P = 8, blocks of 130 rows (ragged against every
    tile).  Contiguous rank 0 sees only its own block (the other seven
    blocks get zeros); rank 7 sees all eight."""
    _check_share(51, 1, 4, 2, 16 * 65, 128, 8, rank, True, layout)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_share_noncausal(d):
    _check_share(52, 2, 2, 1, 4 * 100, d, 4, 1, False, "contiguous")


def test_bwd_share_ragged_small():
    _check_share(53, 1, 2, 1, 3 * 7, 64, 3, 2, True, "striped")


@pytest.mark.parametrize("layout,rank", [("contiguous", 6), ("zigzag", 1)])
def test_bwd_share_fp32(layout, rank):
    _check_share(54, 1, 4, 2, 8 * 34, 64, 8, rank, True, layout, "f32")


def test_bwd_shares_sum_to_the_full_backward():
    """Summed over the P ranks, the shares' dk and dv are the full
    backward's (within the bf16 rounding of the summands), and each rank's
    dq is bitwise the full dq at that rank's rows (the same kv blocks in the
    same order through the same kernel)."""
    import torch
    B, H, Hkv, N, d, P, layout = 1, 4, 2, 8 * 128, 128, 8, "striped"
    q, k, v, do = _inputs(55, B, H, Hkv, N, d, "bf16")
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout)
    dq_f, dk_f, dv_f = (from_dev(t) for t in ra.ring_attn_bwd(qd, kd, vd, out, dod, lse, P=P, causal=True,
                                                                layout=layout))
    dk_sum = np.zeros_like(dk_f)
    dv_sum = np.zeros_like(dv_f)
    for rank, pos in enumerate(oracle.host_positions(N, P, layout)):
        idx = torch.from_numpy(pos).to(qd.device)
        sl = [t.index_select(2, idx).contiguous() for t in (qd, out, dod)]
        dq, dk, dv = ra.ring_attn_bwd_share(sl[0], kd, vd, sl[1], sl[2], lse.index_select(2, idx).contiguous(),
                                            P=P, rank=rank, causal=True, layout=layout)
        torch.cuda.synchronize()
        dq = from_dev(dq)
        assert np.array_equal(dq, dq_f[:, :, pos]), f"rank {rank}: dq differs from ring_attn_bwd"
        dk_sum += from_dev(dk)
        dv_sum += from_dev(dv)
    for got, ref in ((dk_sum, dk_f), (dv_sum, dv_f)):
        assert np.abs(got - ref).max() <= 3e-2 * np.abs(ref).max()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_share_of_one_host_is_the_full_backward(dtype):
    """With P = 1 the one share is the whole backward: bitwise the same
    gradients as ring_attn_bwd (the same kernels over the same rows)."""
    import torch
    B, H, Hkv, N, d = 1, 4, 2, 300, 64
    q, k, v, do = _inputs(56, B, H, Hkv, N, d, dtype)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=1, causal=True)
    full = ra.ring_attn_bwd(qd, kd, vd, out, dod, lse, P=1, causal=True)
    share = ra.ring_attn_bwd_share(qd, kd, vd, out, dod, lse, P=1, rank=0, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(full, share):
        assert np.array_equal(from_dev(a), from_dev(b))


# ---------------------------------------------------------------------------
# The backward building blocks: a ring backward composed on the host from
# ring_attn_bwd_prep and ring_attn_bwd_step over every (query block, kv
# block) pair, with per-block fp32 accumulators, against the oracle.
# ---------------------------------------------------------------------------
def _ring_by_steps(seed, B, H, Hkv, N, d, P, causal, layout, dtype="bf16"):
    import torch
    q, k, v, do = _inputs(seed, B, H, Hkv, N, d, dtype)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=causal, layout=layout)
    pos = oracle.host_positions(N, P, layout)
    idx = [torch.from_numpy(p).to(qd.device) for p in pos]
    blk = lambda t, r: t.index_select(2, idx[r]).contiguous()
    qs = [blk(qd, r) for r in range(P)]
    dos = [blk(dod, r) for r in range(P)]
    ks, vs = [blk(kd, r) for r in range(P)], [blk(vd, r) for r in range(P)]
    rst = [ra.ring_attn_bwd_prep(blk(out, r), dos[r], lse.index_select(2, idx[r]).contiguous()) for r in range(P)]
    Bl = N // P
    f32 = torch.float32
    dq = [torch.zeros((B, H, Bl, d), dtype=f32, device=qd.device) for _ in range(P)]
    dk = [torch.zeros((B, Hkv, Bl, d), dtype=f32, device=qd.device) for _ in range(P)]
    dv = [torch.zeros((B, Hkv, Bl, d), dtype=f32, device=qd.device) for _ in range(P)]
    for s in range(P):          # reverse ring: host r meets kv block (r + s) mod P
        for r in range(P):
            j = (r + s) % P
            ra.ring_attn_bwd_step(qs[r], ks[j], vs[j], dos[r], rst[r], dq[r], dk[j], dv[j], causal=causal,
                                  layout=layout, P=P, q_rank=r, kv_rank=j)
    torch.cuda.synchronize()
    full = [np.zeros((B, H, N, d)), np.zeros((B, Hkv, N, d)), np.zeros((B, Hkv, N, d))]
    for r in range(P):
        full[0][:, :, pos[r]] = from_dev(dq[r])
        full[1][:, :, pos[r]] = from_dev(dk[r])
        full[2][:, :, pos[r]] = from_dev(dv[r])
    return q, k, v, do, full


@pytest.mark.parametrize("layout,causal,dtype", [("contiguous", True, "bf16"), ("striped", True, "bf16"),
                                                 ("zigzag", True, "bf16"), ("contiguous", False, "bf16"),
                                                 ("zigzag", True, "f32")])
def test_bwd_steps_compose_the_ring_backward(layout, causal, dtype):
    """GQA 2:1, d = 128 (64 for fp32), P = 4 ring blocks of 130 rows."""
    d = 128 if dtype == "bf16" else 64
    B, H, Hkv, N, P = 1, 4, 2, 4 * 130, 4
    q, k, v, do, (dq, dk, dv) = _ring_by_steps(57, B, H, Hkv, N, d, P, causal, layout, dtype)
    qh, kh, vh, doh = (host_vals(x, dtype) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    dq_r, dk_r, dv_r, parts = oracle.attention_bwd(qh, kh, vh, doh, scale=scale, causal=causal, parts=True)
    bq, bk, bv = _bounds(qh, kh, vh, doh, parts, B, H, Hkv, scale, dq_r, dk_r, dv_r, EPS[dtype])
    what = f"bwd steps {layout} causal={causal} {dtype}"
    for name, got, ref, bnd in (("dq", dq, dq_r, bq), ("dk", dk, dk_r, bk), ("dv", dv, dv_r, bv)):
        assert np.all(np.isfinite(got)), f"{what}: non-finite {name}"
        err = np.abs(got - ref)
        ratio = float((err / (2 * bnd + 1e-6)).max())
        nw = _normwise(got, ref)
        print(f"  {name}: max|err|={err.max():.3e} normwise={nw:.2e} worst err/bound={ratio:.3f}")
        assert ratio <= 1.0, f"{what}: {name} exceeds its bound (err/bound {ratio:.3f})"
        assert nw <= NORMWISE[dtype], f"{what}: {name} normwise relative error {nw:.2e}"


def test_bwd_step_of_an_invisible_pair_changes_nothing():
    """Contiguous causal: host 0's queries see nothing of kv block 3; the
    step launches nothing and the accumulators keep their values."""
    import torch
    B, H, Hkv, Bl, d, P = 1, 2, 1, 64, 64, 4
    q, k, v, do = _inputs(58, B, H, Hkv, Bl, d, "bf16")
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    rst = torch.zeros((B, H, Bl, 2), dtype=torch.float32, device=qd.device)
    accs = [torch.full((B, H, Bl, d), 7.0, device=qd.device), torch.full((B, Hkv, Bl, d), 7.0, device=qd.device),
            torch.full((B, Hkv, Bl, d), 7.0, device=qd.device)]
    ra.ring_attn_bwd_step(qd, kd, vd, dod, rst, *accs, causal=True, P=P, q_rank=0, kv_rank=3)
    torch.cuda.synchronize()
    for a in accs:
        assert bool((a == 7.0).all())


@pytest.mark.parametrize("layout,dtype", [("contiguous", "bf16"), ("zigzag", "bf16"), ("striped", "f32")])
def test_bwd_steps_are_bitwise_the_ring_backward(layout, dtype):
    """The composed steps add the same products in the same order as
    ring_attn_bwd (its first step writes 0 + x, its last rounds the fp32
    sum once), so rounding their fp32 accumulators like it gives bitwise
    its gradients."""
    import torch
    B, H, Hkv, N, d, P = 1, 4, 2, 4 * 96, 128, 4
    q, k, v, do, (dq, dk, dv) = _ring_by_steps(59, B, H, Hkv, N, d, P, True, layout, dtype)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout)
    ref = ra.ring_attn_bwd(qd, kd, vd, out, dod, lse, P=P, causal=True, layout=layout)
    torch.cuda.synchronize()
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        g = torch.from_numpy(got.astype(np.float32))
        if dtype == "bf16":
            g = g.to(torch.bfloat16)
        assert np.array_equal(from_dev(g), from_dev(r)), f"{name} differs from ring_attn_bwd"
