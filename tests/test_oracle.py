"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than its own formula: a
textbook routine (scipy's logsumexp / softmax without max subtraction),
closed forms, invariants, or the pages' own recurrence and printed figures.
Page cited: "RingAttention 심층 아키텍처" (techknowgenie.com), called [TKG];
sections named inline.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# 1. Brute force on tiny inputs, through a different route: scipy's
#    logsumexp for lse and exp(S - lse) for the weights (no running max,
#    no separate l), loops over every (b, h, i).
# --------------------------------------------------------------------------
def _brute(q, k, v, scale, causal, q_pos, k_pos):
    B, H, Nq, d = q.shape
    Hkv = k.shape[1]
    O = np.zeros((B, H, Nq, v.shape[3]))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            g = (h * Hkv) // H
            for i in range(Nq):
                js = [j for j in range(k.shape[2]) if (not causal) or k_pos[j] <= q_pos[i]]
                if not js:
                    L[b, h, i] = -np.inf
                    continue
                s = np.array([math.fsum(q[b, h, i, c] * k[b, g, j, c] for c in range(d)) * scale
                              for j in js])
                lse = logsumexp(s)
                p = np.exp(s - lse)
                for c in range(v.shape[3]):
                    O[b, h, i, c] = math.fsum(p[t] * v[b, g, js[t], c] for t in range(len(js)))
                L[b, h, i] = lse
    return O, L


@pytest.mark.parametrize("N", [1, 2, 3, 5, 7, 12])
@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("H,Hkv", [(1, 1), (2, 1), (2, 2), (4, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(N, d, H, Hkv, causal):
    rng = np.random.default_rng([N, d, H, Hkv, int(causal)])
    q = _rand(rng, 1, H, N, d) * 2.0
    k = _rand(rng, 1, Hkv, N, d) * 2.0
    v = _rand(rng, 1, Hkv, N, d)
    scale = 1.0 / math.sqrt(d)
    pos = np.arange(N)
    O, L = oracle.attention(q, k, v, scale=scale, causal=causal, threads=2)
    Ob, Lb = _brute(q, k, v, scale, causal, pos, pos)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


def test_brute_force_shifted_positions():
    """Queries at positions 10.. against keys 0..: some rows see all keys."""
    rng = np.random.default_rng(7)
    q = _rand(rng, 2, 2, 5, 3)
    k = _rand(rng, 2, 1, 13, 3)
    v = _rand(rng, 2, 1, 13, 3)
    qp = np.arange(8, 13)
    kp = np.arange(13)
    O, L = oracle.attention(q, k, v, scale=0.7, causal=True, q_pos=qp, k_pos=kp)
    Ob, Lb = _brute(q, k, v, 0.7, True, qp, kp)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(L, Lb, atol=1e-13)


def test_hand_worked_two_keys():
    """q=(1,0), k0=(1,0), k1=(0,1), scale 1: scores (1, 0).

    softmax = (e, 1)/(e+1); O = (e v0 + v1)/(e+1); lse = ln(e+1).
    """
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    O, L = oracle.attention(q, k, v, scale=1.0, causal=False)
    e = math.e
    np.testing.assert_allclose(O[0, 0, 0], [(e * 1 + 3) / (e + 1), (e * 2 + 4) / (e + 1)], atol=1e-15)
    assert abs(L[0, 0, 0] - math.log(e + 1)) < 1e-15


# --------------------------------------------------------------------------
# 2. Softmax normalization: with V = one-hot of the key index, row i of O is
#    the probability row itself; it sums to 1, is >= 0, and is 0 on masked keys.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows(causal):
    rng = np.random.default_rng(11)
    N, d = 9, 3
    q = _rand(rng, 1, 1, N, d) * 3
    k = _rand(rng, 1, 1, N, d) * 3
    v = np.eye(N)[None, None]
    O, L = oracle.attention(q, k, v, scale=0.5, causal=causal)
    P = O[0, 0]
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)
    # and the weights are exp(s - lse) for the textbook lse
    s = (q[0, 0] @ k[0, 0].T) * 0.5
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    np.testing.assert_allclose(P, np.exp(s - logsumexp(s, axis=1, keepdims=True)), atol=1e-14)


# --------------------------------------------------------------------------
# 3. Closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_prefix_mean(causal):
    """Q = 0: all scores 0, so O_i is the mean of V over valid keys and
    lse_i = ln(#valid keys): ln(i + 1) causal, ln N otherwise."""
    rng = np.random.default_rng(3)
    N, d = 17, 5
    q = np.zeros((1, 2, N, d))
    k = _rand(rng, 1, 2, N, d)
    v = _rand(rng, 1, 2, N, d)
    O, L = oracle.attention(q, k, v, scale=1.0, causal=causal)
    for h in range(2):
        for i in range(N):
            n = i + 1 if causal else N
            np.testing.assert_allclose(O[0, h, i], v[0, h, :n].mean(axis=0), atol=1e-14)
            assert abs(L[0, h, i] - math.log(n)) < 1e-14


def test_constant_value_rows():
    """Every row of V equal to c gives O = c whatever Q and K are."""
    rng = np.random.default_rng(5)
    N, d = 11, 4
    q = _rand(rng, 1, 1, N, d) * 5
    k = _rand(rng, 1, 1, N, d) * 5
    c = np.array([0.25, -1.5, 3.0, 7.0])
    v = np.broadcast_to(c, (1, 1, N, d)).copy()
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, scale=1.0, causal=causal)
        np.testing.assert_allclose(O[0, 0], np.broadcast_to(c, (N, d)), atol=1e-13)


def test_single_key():
    """One key: O = v0 and lse = s00."""
    rng = np.random.default_rng(6)
    q = _rand(rng, 1, 1, 1, 8)
    k = _rand(rng, 1, 1, 1, 8)
    v = _rand(rng, 1, 1, 1, 8)
    O, L = oracle.attention(q, k, v, scale=0.3, causal=True)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(L[0, 0, 0] - 0.3 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14


def test_large_logits_stable():
    """Scores around 1e3 stay finite (max subtraction); the result equals
    the same problem with all scores shifted down (softmax shift invariance)."""
    q = np.array([[[[30.0, 0.0], [0.0, 30.0]]]])
    k = np.array([[[[40.0, 0.0], [39.0, 1.0], [0.0, 40.0]]]])
    v = np.array([[[[1.0], [2.0], [3.0]]]])
    O, L = oracle.attention(q, k, v, scale=1.0, causal=False)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    # row 0: scores 1200, 1170, 0 -> weight of key 0 is 1/(1 + e^-30 + e^-1200)
    w1 = math.exp(-30)
    np.testing.assert_allclose(O[0, 0, 0, 0], (1 + 2 * w1) / (1 + w1), rtol=1e-15)
    assert abs(L[0, 0, 0] - (1200 + math.log1p(w1))) < 1e-12


# --------------------------------------------------------------------------
# 4. GQA reading: query head h uses kv head floor(h * Hkv / H), the same as
#    MHA on K/V repeated along the head axis in consecutive groups.
# --------------------------------------------------------------------------
def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(8)
    B, H, Hkv, N, d = 2, 8, 2, 10, 4
    q = _rand(rng, B, H, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    O1, L1 = oracle.attention(q, k, v, causal=True)
    kr = np.repeat(k, H // Hkv, axis=1)
    vr = np.repeat(v, H // Hkv, axis=1)
    O2, L2 = oracle.attention(q, kr, vr, causal=True)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


# --------------------------------------------------------------------------
# 5. lse_merge
# --------------------------------------------------------------------------
def test_lse_merge_closed_forms():
    rng = np.random.default_rng(9)
    oa = _rand(rng, 6, 4)
    ob = _rand(rng, 6, 4)
    la = _rand(rng, 6)
    O, L = oracle.lse_merge(oa, la, ob, la)
    np.testing.assert_allclose(O, (oa + ob) / 2, atol=1e-15)
    np.testing.assert_allclose(L, la + math.log(2), atol=1e-15)
    ninf = np.full(6, -np.inf)
    O, L = oracle.lse_merge(oa, la, ob, ninf)
    np.testing.assert_allclose(O, oa, atol=0)
    np.testing.assert_allclose(L, la, atol=0)
    O, L = oracle.lse_merge(oa, ninf, ob, ninf)
    assert np.all(O == 0) and np.all(L == -np.inf)


def test_lse_merge_of_halves_equals_whole():
    """Attention over keys [0, n) merged from [0, a) and [a, n)."""
    rng = np.random.default_rng(10)
    N, d = 40, 6
    q = _rand(rng, 1, 1, N, d)
    k = _rand(rng, 1, 1, N, d)
    v = _rand(rng, 1, 1, N, d)
    Ow, Lw = oracle.attention(q, k, v, causal=False)
    for a in (1, 13, 39):
        O1, L1 = oracle.attention(q, k[:, :, :a], v[:, :, :a], causal=False)
        O2, L2 = oracle.attention(q, k[:, :, a:], v[:, :, a:], causal=False)
        O, L = oracle.lse_merge(O1, L1, O2, L2)
        np.testing.assert_allclose(O, Ow, atol=1e-13)
        np.testing.assert_allclose(L, Lw, atol=1e-13)


# --------------------------------------------------------------------------
# 6. Decode reading: the single new query sees every cached key; equal to the
#    last row of a causal prefill whose last query is q.
# --------------------------------------------------------------------------
def test_decode_is_last_row_of_causal_prefill():
    rng = np.random.default_rng(12)
    B, H, Hkv, L, d = 2, 4, 2, 23, 8
    k = _rand(rng, B, Hkv, L, d)
    v = _rand(rng, B, Hkv, L, d)
    qfull = _rand(rng, B, H, L, d)
    Od, Ld = oracle.decode(qfull[:, :, -1:], k, v)
    Op, Lp = oracle.attention(qfull, k, v, causal=True)
    np.testing.assert_allclose(Od[:, :, 0], Op[:, :, -1], atol=1e-14)
    np.testing.assert_allclose(Ld[:, :, 0], Lp[:, :, -1], atol=1e-14)


# --------------------------------------------------------------------------
# 7. The pages' central claim: the blockwise ring recurrence of [TKG] §3
#    (m_block, m_new, alpha, beta, l_new, O_new, O_final) reaches the plain
#    definition exactly, for any ring size P, any block order and either
#    layout.  The recurrence is written here from the equations, in the
#    beta form of the page, with the empty-row guard (a row with no valid
#    key in a block leaves its state unchanged).
# --------------------------------------------------------------------------
def _ring_recurrence(q, k, v, scale, causal, P, layout, order):
    N, d = q.shape
    pos = oracle.host_positions(N, P, layout)
    O = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for r in range(P):
        qi = q[pos[r]]
        m = np.full(len(pos[r]), -np.inf)
        l = np.zeros(len(pos[r]))
        acc = np.zeros((len(pos[r]), v.shape[1]))
        for kv in order(r):
            S = (qi @ k[pos[kv]].T) * scale
            if causal:
                S = np.where(pos[kv][None, :] <= pos[r][:, None], S, -np.inf)
            m_blk = S.max(axis=1)
            m_new = np.maximum(m, m_blk)
            live = np.isfinite(m_new)
            m_new_s = np.where(live, m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - m_new_s), 0.0)
            blk_live = np.isfinite(m_blk)
            m_blk_s = np.where(blk_live, m_blk, 0.0)
            beta = np.where(blk_live, np.exp(m_blk_s - m_new_s), 0.0)
            Pc = np.where(np.isfinite(S), np.exp(S - m_blk_s[:, None]), 0.0)
            l = l * alpha + Pc.sum(axis=1) * beta
            acc = acc * alpha[:, None] + (Pc @ v[pos[kv]]) * beta[:, None]
            m = np.where(live, m_new, m)
        O[pos[r]] = acc / l[:, None]
        lse[pos[r]] = m + np.log(l)
    return O, lse


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("causal", [False, True])
def test_ring_recurrence_reaches_oracle(P, layout, causal):
    rng = np.random.default_rng([P, int(causal), len(layout)])
    N, d = 64, 8
    q = _rand(rng, N, d)
    k = _rand(rng, N, d)
    v = _rand(rng, N, d)
    Oo, Lo = oracle.attention(q[None, None], k[None, None], v[None, None], causal=causal)
    # ring order of [TKG] §5: at step s host r holds block (r - s) mod P
    Or, Lr = _ring_recurrence(q, k, v, 1 / math.sqrt(d), causal, P, layout,
                              lambda r: [(r - s) % P for s in range(P)])
    np.testing.assert_allclose(Or, Oo[0, 0], atol=1e-12)
    np.testing.assert_allclose(Lr, Lo[0, 0], atol=1e-12)
    # any other block order gives the same result
    perm_rng = np.random.default_rng(P)
    perms = [list(perm_rng.permutation(P)) for _ in range(3)]
    for perm in perms:
        Or2, Lr2 = _ring_recurrence(q, k, v, 1 / math.sqrt(d), causal, P, layout, lambda r: perm)
        np.testing.assert_allclose(Or2, Oo[0, 0], atol=1e-12)
        np.testing.assert_allclose(Lr2, Lo[0, 0], atol=1e-12)


def test_step_partial_matches_recurrence_pieces():
    """step_partial returns the block's (m_block, l_curr, P_curr V) of [TKG] §3."""
    rng = np.random.default_rng(13)
    q = _rand(rng, 6, 4)
    k = _rand(rng, 9, 4)
    v = _rand(rng, 9, 4)
    qp = np.array([3, 5, 7, 9, 11, 13])
    kp = np.arange(0, 18, 2)
    m, l, o, lse, On = oracle.step_partial(q, k, v, scale=0.5, causal=True, q_pos=qp, k_pos=kp)
    S = (q @ k.T) * 0.5
    valid = kp[None, :] <= qp[:, None]
    for i in range(6):
        s = S[i][valid[i]]
        assert m[i] == s.max()
        w = np.exp(s - s.max())
        np.testing.assert_allclose(l[i], w.sum(), rtol=1e-15)
        np.testing.assert_allclose(o[i], w @ v[valid[i]], atol=1e-13)
        np.testing.assert_allclose(lse[i], logsumexp(s), atol=1e-14)


def test_step_partial_empty_rows():
    """A query row with no valid key in the block: m = lse = -inf, l = 0, o = 0."""
    q = np.ones((2, 3))
    k = np.ones((4, 3))
    v = np.ones((4, 3))
    m, l, o, lse, On = oracle.step_partial(q, k, v, scale=1.0, causal=True,
                                           q_pos=np.array([0, 10]), k_pos=np.array([5, 6, 7, 8]))
    assert m[0] == -np.inf and l[0] == 0 and np.all(o[0] == 0) and lse[0] == -np.inf
    assert np.isfinite(m[1]) and l[1] == pytest.approx(4.0)


# --------------------------------------------------------------------------
# 8. Layout and work counts, pinned to the pages' figures.
# --------------------------------------------------------------------------
def test_host_positions_partition():
    for layout in ("contiguous", "striped", "zigzag"):
        pos = oracle.host_positions(24, 4, layout)
        allp = np.sort(np.concatenate(pos))
        np.testing.assert_array_equal(allp, np.arange(24))
        # positions inside a block increase with the row (the kernels rely on it)
        for p in pos:
            assert np.all(np.diff(p) > 0)
    assert list(oracle.host_positions(8, 4, "striped")[1]) == [1, 5]
    assert list(oracle.host_positions(8, 4, "contiguous")[1]) == [2, 3]
    # zigzag, 2P = 4 chunks of 2: host 0 pairs the first and last chunk
    assert list(oracle.host_positions(8, 2, "zigzag")[0]) == [0, 1, 6, 7]
    assert list(oracle.host_positions(8, 2, "zigzag")[1]) == [2, 3, 4, 5]
    with pytest.raises(ValueError):
        oracle.host_positions(12, 4, "zigzag")


@pytest.mark.parametrize("P,N", [(4, 32), (8, 64), (8, 256)])
def test_pair_counts_closed_forms(P, N):
    Bl = N // P
    st = oracle.pair_counts(N, P, "striped", causal=True)
    for rq, rk in itertools.product(range(P), repeat=2):
        want = Bl * (Bl + 1) // 2 if rk <= rq else Bl * (Bl - 1) // 2
        assert st[rq, rk] == want
    co = oracle.pair_counts(N, P, "contiguous", causal=True)
    for rq, rk in itertools.product(range(P), repeat=2):
        want = Bl * Bl if rk < rq else (Bl * (Bl + 1) // 2 if rk == rq else 0)
        assert co[rq, rk] == want
    assert st.sum() == co.sum() == N * (N + 1) // 2
    # striped: every host gets the same total share of the causal triangle ([TKG] §7)
    rows = st.sum(axis=1)
    assert rows.max() - rows.min() <= P * Bl
    # zigzag: 2C^2 + C on the diagonal block, 2C^2 on every other block, so
    # every host's share is exactly the same
    C = N // (2 * P)
    zz = oracle.pair_counts(N, P, "zigzag", causal=True)
    for rq, rk in itertools.product(range(P), repeat=2):
        assert zz[rq, rk] == (2 * C * C + C if rk == rq else 2 * C * C)
    assert zz.sum() == N * (N + 1) // 2
    assert len(set(zz.sum(axis=1))) == 1


def test_pages_printed_figures():
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    sm = g["score_matrix_1M"]
    assert sm["N"] ** 2 == sm["elements"]
    assert sm["elements"] * sm["bytes_per_element_fp16"] == sm["bytes"]
    # a full (non-causal) block pair of B tokens holds B^2 unmasked pairs; at
    # 4 d FLOPs per pair this is the page's 4 B^2 d block compute figure
    zb = g["zero_bubble_table"]
    B, P = 64, 4
    pc = oracle.pair_counts(B * P, P, "contiguous", causal=False)
    d = 128
    assert int(pc[0, 1]) * 4 * d == zb["flops_per_block_pair_coeff"] * B * B * d


# --------------------------------------------------------------------------
# 9. The synthetic generator: bf16 rounding is round-to-nearest-even.
# --------------------------------------------------------------------------
def test_bf16_rounding_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 1.0 + 2 ** -7 + 2 ** -9],
                 dtype=np.float32)
    bits = synth.bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even -> 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    np.testing.assert_array_equal(back, np.array(
        [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 1.0 + 2 ** -7], dtype=np.float32))


def test_synth_slab_reproducible():
    a = synth.tensor(1, synth.TENSOR_K, 2, 3, 16, 8, "bf16", threads=1)
    b = synth.tensor(1, synth.TENSOR_K, 2, 3, 16, 8, "bf16", threads=4)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a[1, 2], synth.slab_bits(1, synth.TENSOR_K, 1, 2, 16, 8))


def test_synth_uniform_range_and_reproducible():
    a = synth.uniform_tensor(4, synth.TENSOR_V, 2, 3, 50, 8, 2.0, 3.9, "bf16")
    b = synth.uniform_tensor(4, synth.TENSOR_V, 2, 3, 50, 8, 2.0, 3.9, "bf16")
    np.testing.assert_array_equal(a, b)
    x = synth.as_f32(a, "bf16")
    assert x.min() >= 2.0 and x.max() <= 3.9 + 2 ** -6   # bf16 rounding of values below 3.9
    f = synth.uniform_tensor(4, synth.TENSOR_V, 2, 3, 50, 8, 2.0, 3.9, "f32")
    np.testing.assert_array_equal(synth.bf16_bits(f), a)
