"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Small and ragged shapes that span several 128-row query tiles and 64-key
tiles plus a tail; every call goes through the C ABI (via the ctypes
binding).  Tolerances: fp32 max|dO|, max|dlse| <= 1e-5; bf16 max|dO| <= 1e-2,
max|dlse| <= 1e-3.
"""
import math

import numpy as np
import pytest

import blockwise_ring_attention_attn_amd as ra
import oracle
import synth
from _util import assert_close, from_dev, host_vals, max_err, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, B, H, Hkv, N, d, dtype, Nq=None):
    print(f"\n[case] seed={seed} B={B} H={H} Hkv={Hkv} N={N} d={d} dtype={dtype} Nq={Nq}", flush=True)
    return synth.qkv(seed, B, H, Hkv, N, d, dtype, Nq=Nq)


def _fwd_and_check(seed, B, H, Hkv, N, d, P, causal, layout, dtype):
    q, k, v = _case(seed, B, H, Hkv, N, d, dtype)
    out, lse = ra.ring_attn_fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), P=P, causal=causal,
                                layout=layout)
    import torch
    torch.cuda.synchronize()
    Ow, Lw = oracle.attention(host_vals(q, dtype), host_vals(k, dtype), host_vals(v, dtype),
                              scale=1 / math.sqrt(d), causal=causal)
    return assert_close(from_dev(out), from_dev(lse), Ow, Lw, dtype,
                        f"fwd B={B} H={H}/{Hkv} N={N} d={d} P={P} causal={causal} {layout} {dtype}")


def test_config1_fp32_noncausal_P4():
    """Single head, N=1024, d=64, fp32, non-causal, P=4 ring blocks of 256."""
    eo, el = _fwd_and_check(1, 1, 1, 1, 1024, 64, 4, False, "contiguous", "f32")
    print(f"config1 max|dO|={eo:.2e} max|dlse|={el:.2e}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_fp32_small(d, causal, layout):
    _fwd_and_check(7, 1, 2, 1, 4 * 75, d, 4, causal, layout, "f32")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_small_zigzag(d, causal):
    """Zigzag: 2P = 8 chunks of 75 tokens (ragged against every tile size)."""
    _fwd_and_check(7, 1, 2, 1, 8 * 75, d, 4, causal, "zigzag", "f32")


@pytest.mark.parametrize("N,P", [(8, 8), (24, 8), (8 * 130, 8), (4 * 257, 4), (3 * 384, 3), (700, 1)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_bf16_causal_ragged(N, P, d, layout):
    _fwd_and_check(2, 1, 4, 2, N, d, P, True, layout, "bf16")


# zigzag needs N % 2P == 0; chunks of 1, 3, 130, 257 and 384 tokens, and P = 1
@pytest.mark.parametrize("N,P", [(16, 8), (48, 8), (16 * 130, 8), (8 * 257, 4), (6 * 384, 3), (700, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_causal_ragged_zigzag(N, P, d):
    _fwd_and_check(2, 1, 4, 2, N, d, P, True, "zigzag", "bf16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_bf16_large_outputs_few_keys(d, layout):
    """Values drawn from U(2, 3.9), so every output lies in [2, 3.9], where
    one bf16 ulp is 2^-6 and rounding the output alone costs up to 0.0078.
    The rows with 1-8 keys (the first rows of the sequence; in the striped
    layout the first row of every host block) leave about 0.002 for the
    kernel's own error.  Dividing by the sum of the bf16 weights the P V
    product applies keeps that error proportional to the spread of the
    values; dividing by the fp32 weight sum would scale it with the values
    (up to 2^-8 * 3.9 = 0.015)."""
    import torch
    B, H, Hkv, N, P = 1, 4, 2, 8 * 130, 8
    q, k, _ = _case(11, B, H, Hkv, N, d, "bf16")
    v = synth.uniform_tensor(11, synth.TENSOR_V, B, Hkv, N, d, 2.0, 3.9, "bf16")
    out, lse = ra.ring_attn_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), P=P, causal=True,
                                layout=layout)
    torch.cuda.synchronize()
    Ow, Lw = oracle.attention(host_vals(q, "bf16"), host_vals(k, "bf16"), host_vals(v, "bf16"),
                              scale=1 / math.sqrt(d), causal=True)
    assert Ow.min() >= 2.0 and Ow.max() <= 3.9
    eo, el = assert_close(from_dev(out), from_dev(lse), Ow, Lw, "bf16", f"large outputs d={d} {layout}")
    print(f"large outputs d={d} {layout}: max|dO|={eo:.2e} max|dlse|={el:.2e}")


@pytest.mark.parametrize("rise", [60.0, -60.0])
def test_scores_rising_or_falling_along_the_keys(rise):
    """Scores that grow (or shrink) by about 60 natural units along the keys:
    q_i = x_i + a u and k_j = y_j + b_j u for a unit vector u and b_j linear
    in j.  When they grow, a row's weights against its reference max keep
    outgrowing the accepted range, so the bf16 kernel moves its reference
    many times in mid-row (and at tiles that are not the first); when they
    fall, every later tile underflows against the first one's max.  Either
    way the result must match the oracle.  (bf16 only: the fp32 kernel keeps
    the exact running max, and with |lse| near 34 the absolute fp32 bound of
    1e-5 is about three fp32 ulps of lse itself.)"""
    import torch
    dtype = "bf16"
    B, H, Hkv, N, d, P = 1, 2, 1, 4 * 300, 128, 4
    q, k, v = _case(13, B, H, Hkv, N, d, dtype)
    rng = np.random.default_rng([13, 99])
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    a = 8.0
    b = rise * math.sqrt(d) / a * (np.arange(N) / (N - 1) - 0.5)
    qf = synth.bf16_bits((host_vals(q, dtype) + a * u).astype(np.float32))
    kf = synth.bf16_bits((host_vals(k, dtype) + b[None, None, :, None] * u).astype(np.float32))
    q2, k2 = to_dev(qf, dtype), to_dev(kf, dtype)
    out, lse = ra.ring_attn_fwd(q2, k2, to_dev(v, dtype), P=P, causal=True, layout="contiguous")
    torch.cuda.synchronize()
    qh, kh = from_dev(q2), from_dev(k2)
    S_span = (qh[0, 0] @ kh[0, 0].T / math.sqrt(d))
    print(f"score range along row {N - 1}: {S_span[-1].min():.1f} .. {S_span[-1].max():.1f}")
    Ow, Lw = oracle.attention(qh, kh, host_vals(v, dtype), scale=1 / math.sqrt(d), causal=True)
    assert_close(from_dev(out), from_dev(lse), Ow, Lw, dtype, f"rise={rise}")


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_batched_gqa(causal):
    _fwd_and_check(3, 2, 8, 2, 4 * 320, 128, 4, causal, "contiguous", "bf16")


def test_bf16_layout_and_P_invariance():
    """Same inputs: contiguous P=8, striped P=8 and P=2, P=1, zigzag P=8 and
    P=2 agree with each other within twice the tolerance."""
    dtype, N, d = "bf16", 8 * 256, 128
    q, k, v = _case(4, 1, 2, 2, N, d, dtype)
    outs = []
    for layout, P in (("contiguous", 8), ("striped", 8), ("striped", 2), ("contiguous", 1), ("zigzag", 8),
                      ("zigzag", 2)):
        o, l = ra.ring_attn_fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), P=P, causal=True,
                                layout=layout)
        outs.append((from_dev(o), from_dev(l)))
    for o, l in outs[1:]:
        assert max_err(o, outs[0][0]) <= 2e-2 and max_err(l, outs[0][1]) <= 2e-3


def test_gqa_equals_repeated_kv_bitwise():
    dtype, N, d = "bf16", 4 * 200, 64
    q, k, v = _case(5, 1, 4, 2, N, d, dtype)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    o1, l1 = ra.ring_attn_fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), P=4, causal=True)
    o2, l2 = ra.ring_attn_fwd(to_dev(q, dtype), to_dev(kr, dtype), to_dev(vr, dtype), P=4, causal=True)
    assert np.array_equal(from_dev(o1), from_dev(o2)) and np.array_equal(from_dev(l1), from_dev(l2))


def test_deterministic_bitwise():
    dtype, N, d = "bf16", 8 * 300, 128
    q, k, v = _case(6, 1, 4, 4, N, d, dtype)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    r1 = ra.ring_attn_fwd(qd, kd, vd, P=8, causal=True, layout="striped")
    r2 = ra.ring_attn_fwd(qd, kd, vd, P=8, causal=True, layout="striped")
    assert np.array_equal(from_dev(r1[0]), from_dev(r2[0]))
    assert np.array_equal(from_dev(r1[1]), from_dev(r2[1]))


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_share_matches_oracle(layout, dtype):
    """One host's share: q holds host `rank`'s tokens, k, v the whole sequence."""
    import torch
    B, H, Hkv, N, d, P = 1, 4, 2, 8 * 192, 128, 8
    q, k, v = _case(8, B, H, Hkv, N, d, dtype)
    pos = oracle.host_positions(N, P, layout)
    for rank in (0, 3, 7):
        qr = np.ascontiguousarray(q[:, :, pos[rank]])
        o, l = ra.ring_attn_fwd_share(to_dev(qr, dtype), to_dev(k, dtype), to_dev(v, dtype), P=P, rank=rank,
                                      causal=True, layout=layout)
        torch.cuda.synchronize()
        Ow, Lw = oracle.attention(host_vals(qr, dtype), host_vals(k, dtype), host_vals(v, dtype),
                                  causal=True, q_pos=pos[rank])
        assert_close(from_dev(o), from_dev(l), Ow, Lw, dtype, f"share rank={rank} {layout}")


@pytest.mark.parametrize("layout,dtype", [("contiguous", "bf16"), ("striped", "bf16"), ("zigzag", "bf16"),
                                          ("striped", "f32")])
def test_shares_assemble_the_full_ring_bitwise(layout, dtype):
    """The P shares, each rank's queries against every kv block in its ring
    order, run the same kernel over the same blocks in the same order as
    the full ring does for that host: put back at their positions, their
    outputs and lse are bitwise those of ring_attn_fwd."""
    import torch
    B, H, Hkv, N, d, P = 1, 4, 2, 8 * 160, 128, 8
    q, k, v = _case(10, B, H, Hkv, N, d, dtype)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout)
    torch.cuda.synchronize()
    out, lse = from_dev(out), from_dev(lse)
    for rank, pos in enumerate(oracle.host_positions(N, P, layout)):
        o, l = ra.ring_attn_fwd_share(to_dev(np.ascontiguousarray(q[:, :, pos]), dtype), kd, vd, P=P, rank=rank,
                                      causal=True, layout=layout)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(o), out[:, :, pos]), f"rank {rank}: output differs"
        assert np.array_equal(from_dev(l), lse[:, :, pos]), f"rank {rank}: lse differs"


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_state_against_oracle(layout, dtype):
    """ring_attn_step on one (q block, kv block) pair, then on a second kv
    block: lse = m + ln l and O = o / l match the oracle's partial over the
    keys seen; m stays within 16/log2(e) below the true max."""
    import torch
    B, H, Hkv, N, d, P = 1, 2, 1, 4 * 200, 64, 4
    q, k, v = _case(9, B, H, Hkv, N, d, dtype)
    pos = oracle.host_positions(N, P, layout)
    qr, kr_ = 2, 1
    qb = np.ascontiguousarray(q[:, :, pos[qr]])
    m, l, o = ra.init_state(B, H, N // P, d, "cuda:0")
    seen = []
    for kvr in (kr_, qr):
        kb = np.ascontiguousarray(k[:, :, pos[kvr]])
        vb = np.ascontiguousarray(v[:, :, pos[kvr]])
        ra.ring_attn_step(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), m, l, o, causal=True,
                          layout=layout, P=P, q_rank=qr, kv_rank=kvr)
        seen.append(kvr)
        torch.cuda.synchronize()
        kp = np.concatenate([pos[r] for r in seen])
        ks = np.concatenate([host_vals(k, dtype)[:, :, pos[r]] for r in seen], axis=2)
        vs = np.concatenate([host_vals(v, dtype)[:, :, pos[r]] for r in seen], axis=2)
        Ow, Lw = oracle.attention(host_vals(qb, dtype), ks, vs, causal=True, q_pos=pos[qr], k_pos=kp)
        mh, lh, oh = from_dev(m), from_dev(l), from_dev(o)
        with np.errstate(divide="ignore", invalid="ignore"):
            lse = mh + np.log(lh)
            On = np.where(lh[..., None] > 0, oh / lh[..., None], 0.0)
        assert_close(On, lse, Ow, Lw, dtype, f"step kv={seen}")
        # the stored m is a valid reference: never above the true max, at most 16/log2 e below
        S = np.einsum("bhid,bhjd->bhij", host_vals(qb, dtype).astype(np.float64),
                      np.repeat(ks, H // Hkv, axis=1).astype(np.float64)) / math.sqrt(d)
        S = np.where(kp[None, None, None, :] <= pos[qr][None, None, :, None], S, -np.inf)
        true_max = S.max(axis=-1)
        fin = np.isfinite(true_max)
        assert np.all(mh[fin] <= true_max[fin] + 1e-4)
        assert np.all(mh[fin] >= true_max[fin] - 16 / math.log2(math.e) - 1e-4)
        assert np.all(np.isneginf(mh[~fin]))


def test_step_then_finalize_and_empty_rows():
    """Striped causal step with kv_rank > q_rank: row 0 sees no key, so its
    state stays (m=-inf, l=0, o=0) and finalize gives O=0, lse=-inf."""
    import torch
    dtype, B, H, N, d, P = "bf16", 1, 1, 4 * 64, 64, 4
    q, k, v = _case(10, B, H, H, N, d, dtype)
    pos = oracle.host_positions(N, P, "striped")
    qb = np.ascontiguousarray(q[:, :, pos[1]])
    kb = np.ascontiguousarray(k[:, :, pos[3]])
    vb = np.ascontiguousarray(v[:, :, pos[3]])
    m, l, o = ra.init_state(B, H, N // P, d, "cuda:0")
    ra.ring_attn_step(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), m, l, o, causal=True,
                      layout="striped", P=P, q_rank=1, kv_rank=3)
    out, lse = ra.ring_attn_finalize(m, l, o, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Ow, Lw = oracle.attention(host_vals(qb, dtype), host_vals(kb, dtype), host_vals(vb, dtype), causal=True,
                              q_pos=pos[1], k_pos=pos[3])
    assert from_dev(l)[0, 0, 0] == 0 and np.isneginf(from_dev(lse)[0, 0, 0])
    assert np.all(from_dev(out)[0, 0, 0] == 0)
    assert_close(from_dev(out), from_dev(lse), Ow, Lw, dtype, "step+finalize")


def test_merge_and_finalize_of_empty_inputs():
    """Zero rows: both calls return without launching, leaving nothing to check but that they succeed."""
    import torch
    oa = torch.empty((0, 64), device="cuda:0")
    la = torch.empty((0,), device="cuda:0")
    ra.lse_merge(oa, la, oa.clone(), la.clone())
    m, l, o = ra.init_state(1, 1, 0, 64, "cuda:0")
    out, lse = ra.ring_attn_finalize(m, l, o, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert out.shape == (1, 1, 0, 64) and lse.shape == (1, 1, 0)


def test_lse_merge_against_oracle():
    import torch
    rng = np.random.default_rng(11)
    rows, d = 1000, 96
    oa, ob = rng.standard_normal((rows, d)).astype(np.float32), rng.standard_normal((rows, d)).astype(np.float32)
    la, lb = (rng.standard_normal(rows) * 5).astype(np.float32), (rng.standard_normal(rows) * 5).astype(np.float32)
    la[:10] = -np.inf
    lb[5:15] = -np.inf
    Ow, Lw = oracle.lse_merge(oa, la, ob, lb)
    ta, tla = torch.from_numpy(oa).cuda(), torch.from_numpy(la).cuda()
    ra.lse_merge(ta, tla, torch.from_numpy(ob).cuda(), torch.from_numpy(lb).cuda())
    torch.cuda.synchronize()
    assert max_err(from_dev(ta), Ow) <= 1e-5 and max_err(from_dev(tla), Lw) <= 1e-5
    assert np.all(from_dev(ta)[5:10] == 0) and np.all(np.isneginf(from_dev(tla)[5:10]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,Hkv,L,d,P", [(2, 8, 2, 8 * 1000, 128, 8), (3, 4, 4, 4 * 77, 64, 4),
                                           (1, 16, 1, 2 * 4096, 128, 2), (2, 2, 2, 1, 128, 1),
                                           (2, 32, 1, 4 * 512, 128, 4), (1, 40, 2, 8 * 300, 64, 8)])
def test_decode_against_oracle(B, H, Hkv, L, d, P, dtype):
    """Decode against the oracle, including multi-query attention (32 query
    heads on one kv head: two sub-groups of 16) and a group of 20 (a full
    sub-group and one of 4)."""
    import torch
    q, k, v = _case(12, B, H, Hkv, L, d, dtype, Nq=1)
    out, lse = ra.ring_attn_decode(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), P=P)
    torch.cuda.synchronize()
    Ow, Lw = oracle.decode(host_vals(q, dtype), host_vals(k, dtype), host_vals(v, dtype))
    assert_close(from_dev(out), from_dev(lse), Ow, Lw[:, :, 0], dtype, f"decode B={B} H={H}/{Hkv} L={L} {dtype}")


@pytest.mark.parametrize("L,P", [(24, 8), (200, 4), (1000, 8)])
def test_decode_large_outputs(L, P):
    """Decode with values from U(2, 3.9) and short caches (3 to 125 keys per
    ring block): every output lies in [2, 3.9] (see
    test_bf16_large_outputs_few_keys)."""
    import torch
    B, H, Hkv, d = 2, 8, 2, 128
    q, k, _ = _case(13, B, H, Hkv, L, d, "bf16", Nq=1)
    v = synth.uniform_tensor(13, synth.TENSOR_V, B, Hkv, L, d, 2.0, 3.9, "bf16")
    out, lse = ra.ring_attn_decode(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), P=P)
    torch.cuda.synchronize()
    Ow, Lw = oracle.decode(host_vals(q, "bf16"), host_vals(k, "bf16"), host_vals(v, "bf16"))
    assert_close(from_dev(out), from_dev(lse), Ow, Lw[:, :, 0], "bf16", f"decode large outputs L={L} P={P}")


def test_decode_P1_equals_P8():
    import torch
    dtype = "bf16"
    q, k, v = _case(13, 2, 8, 2, 8 * 512, 128, dtype, Nq=1)
    r1 = ra.ring_attn_decode(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), P=1)
    r8 = ra.ring_attn_decode(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), P=8)
    torch.cuda.synchronize()
    assert max_err(from_dev(r1[0]), from_dev(r8[0])) <= 1e-2
    assert max_err(from_dev(r1[1]), from_dev(r8[1])) <= 1e-4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_states_merge_by_the_pages_update(dtype):
    """Two ring_attn_step states over disjoint kv blocks, merged on the host
    by the [TKG] §3 update (m_new = max(m_a, m_b), alpha = e^(m_a - m_new),
    beta = e^(m_b - m_new), l = alpha l_a + beta l_b, o = alpha o_a + beta
    o_b), give the attention over both blocks: the stored m (a reference
    max, possibly below the true max) carries l and o consistently."""
    import torch
    B, H, Hkv, N, d, P = 1, 2, 1, 4 * 192, 128, 4
    q, k, v = _case(14, B, H, Hkv, N, d, dtype)
    pos = oracle.host_positions(N, P, "contiguous")
    qr = 3
    qb = np.ascontiguousarray(q[:, :, pos[qr]])
    states = []
    for kvr in (1, 3):
        kb = np.ascontiguousarray(k[:, :, pos[kvr]])
        vb = np.ascontiguousarray(v[:, :, pos[kvr]])
        m, l, o = ra.init_state(B, H, N // P, d, "cuda:0")
        ra.ring_attn_step(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), m, l, o, causal=True,
                          layout="contiguous", P=P, q_rank=qr, kv_rank=kvr)
        torch.cuda.synchronize()
        states.append(tuple(from_dev(t).astype(np.float64) for t in (m, l, o)))
    (ma, la, oa), (mb, lb, ob) = states
    m_new = np.maximum(ma, mb)
    alpha, beta = np.exp(ma - m_new), np.exp(mb - m_new)
    l_new = alpha * la + beta * lb
    o_new = alpha[..., None] * oa + beta[..., None] * ob
    kp = np.concatenate([pos[1], pos[3]])
    ks = np.concatenate([host_vals(k, dtype)[:, :, pos[r]] for r in (1, 3)], axis=2)
    vs = np.concatenate([host_vals(v, dtype)[:, :, pos[r]] for r in (1, 3)], axis=2)
    Ow, Lw = oracle.attention(host_vals(qb, dtype), ks, vs, causal=True, q_pos=pos[qr], k_pos=kp)
    assert_close(o_new / l_new[..., None], m_new + np.log(l_new), Ow, Lw, dtype, "pages' merge of two states")
