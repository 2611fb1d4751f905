"""Pins of the fp64 backward oracle (oracle/backward.py) against things other
than itself: central finite differences of the (separately pinned) forward
oracle, exact invariants of the softmax Jacobian, special cases with closed
forms, and the grouped-query identity.  CPU only.
"""

import numpy as np
import pytest

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, dO, **kw):
    O, _ = oracle.attention(q, k, v, **kw)
    return float((O * dO).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("positions", [False, True])
def test_matches_finite_differences(causal, positions):
    """Every gradient entry equals the central difference of
    L = sum(O * dO) computed with the forward oracle."""
    rng = np.random.default_rng([31, int(causal), int(positions)])
    B, H, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    dO = _rand(rng, B, H, N, d)
    kw = dict(scale=0.7, causal=causal)
    if positions:  # striped-like positions, queries and keys interleaved
        kw.update(q_pos=np.array([1, 3, 5, 7, 9]), k_pos=np.array([0, 2, 4, 6, 8]))
    dq, dk, dv = oracle.attention_bwd(q, k, v, dO, **kw)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], dO, **kw)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], dO, **kw)
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, atol=2e-8, rtol=0, err_msg=name)


def test_softmax_jacobian_invariants():
    """Each row of dS sums to zero (softmax rows sum to one), so the keys'
    dK sum to zero; dV summed over keys equals dO summed over queries."""
    rng = np.random.default_rng(32)
    B, H, Hkv, N, d = 2, 4, 2, 23, 8
    q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    dO = _rand(rng, B, H, N, d)
    dq, dk, dv, parts = oracle.attention_bwd(q, k, v, dO, causal=True, parts=True)
    for (b, h), p in parts.items():
        np.testing.assert_allclose(p["dS"].sum(axis=1), 0.0, atol=1e-13)
        np.testing.assert_allclose(p["P"].sum(axis=1), 1.0, atol=1e-14)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    group = H // Hkv
    dO_g = dO.reshape(B, Hkv, group, N, d).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), dO_g.sum(axis=2), atol=1e-12)


def test_single_key_and_zero_upstream():
    rng = np.random.default_rng(33)
    q, k, v = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 1, 1, 3), _rand(rng, 1, 1, 1, 3)
    dO = _rand(rng, 1, 2, 4, 3)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dO)
    # one key: P = 1 everywhere, so dS = 0 and dV collects all of dO
    assert np.all(dq == 0) and np.allclose(dk, 0, atol=1e-15)
    np.testing.assert_allclose(dv[0, 0, 0], dO[0].sum(axis=(0, 1)), atol=1e-14)
    z = oracle.attention_bwd(q, k, v, np.zeros_like(dO))
    assert all(np.all(t == 0) for t in z)


def test_rows_without_visible_keys_contribute_nothing():
    rng = np.random.default_rng(34)
    q, k, v = _rand(rng, 1, 1, 3, 4), _rand(rng, 1, 1, 5, 4), _rand(rng, 1, 1, 5, 4)
    dO = _rand(rng, 1, 1, 3, 4)
    qp, kp = np.array([0, 10, 20]), np.array([5, 6, 7, 8, 9])
    dq, dk, dv = oracle.attention_bwd(q, k, v, dO, causal=True, q_pos=qp, k_pos=kp)
    assert np.all(dq[0, 0, 0] == 0)
    # the same as dropping query row 0
    dq2, dk2, dv2 = oracle.attention_bwd(q[:, :, 1:], k, v, dO[:, :, 1:], causal=True, q_pos=qp[1:], k_pos=kp)
    np.testing.assert_allclose(dk, dk2, atol=1e-14)
    np.testing.assert_allclose(dv, dv2, atol=1e-14)
    np.testing.assert_allclose(dq[:, :, 1:], dq2, atol=1e-14)


def test_gqa_equals_repeated_kv_summed():
    rng = np.random.default_rng(35)
    B, H, Hkv, N, d = 1, 4, 2, 9, 5
    q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    dO = _rand(rng, B, H, N, d)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dO, causal=True)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = oracle.attention_bwd(q, kr, vr, dO, causal=True)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, 2, N, d).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, 2, N, d).sum(axis=2), atol=1e-13)


def test_layout_invariance_through_positions():
    """Permuting the token order (with positions carried along) permutes the
    gradients the same way: the gradient does not depend on the layout."""
    rng = np.random.default_rng(36)
    N, d, P = 16, 4, 4
    q, k, v = _rand(rng, 1, 1, N, d), _rand(rng, 1, 1, N, d), _rand(rng, 1, 1, N, d)
    dO = _rand(rng, 1, 1, N, d)
    ref = oracle.attention_bwd(q, k, v, dO, causal=True)
    for layout in ("striped", "zigzag"):
        order = np.concatenate(oracle.host_positions(N, P, layout))
        got = oracle.attention_bwd(q[:, :, order], k[:, :, order], v[:, :, order], dO[:, :, order], causal=True,
                                   q_pos=order, k_pos=order)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b[:, :, order], atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [7, 64])
def test_sampled_gradients_equal_full(causal, chunk):
    """The sampled form (one head, chunked, no [N, N] matrix) gives the same
    rows of dq and the same key rows of dk, dv as the full evaluation, for a
    head whose kv head has one query head (H == Hkv)."""
    rng = np.random.default_rng([37, int(causal), chunk])
    B, H, N, d = 2, 3, 130, 8
    q, k, v, dO = (_rand(rng, B, H, N, d) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, dO, causal=causal, scale=0.4)
    rows = np.array([0, 1, 63, 64, 129])
    keys = np.array([0, 5, 127, 129])
    for (b, h) in ((0, 0), (1, 2)):
        dqr, dkk, dvk, parts = oracle.attention_bwd_sampled(q, k, v, dO, b=b, h=h, rows=rows, keys=keys,
                                                             scale=0.4, causal=causal, chunk=chunk)
        np.testing.assert_allclose(dqr, dq[b, h, rows], atol=1e-12)
        np.testing.assert_allclose(dkk, dk[b, h, keys], atol=1e-12)
        np.testing.assert_allclose(dvk, dv[b, h, keys], atol=1e-12)
        O, lse = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale=0.4,
                                  causal=causal)
        np.testing.assert_allclose(parts["O"], O[0, 0], atol=1e-12)
        np.testing.assert_allclose(parts["lse"], lse[0, 0], atol=1e-12)


def test_row_subset_gives_its_rows_and_the_keys_only_they_see():
    """The full-size backward tests evaluate the oracle on a subset of query
    rows at their positions: each row's softmax depends on no other row, so
    the subset's dq equals the full dq at those rows, and the subset's dk, dv
    of keys that only those rows see (causal: the last keys) equal the full
    ones, with GQA's query heads of a kv head summed."""
    rng = np.random.default_rng(38)
    B, H, Hkv, N, d = 1, 4, 2, 96, 8
    q, dO = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    k, v = _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dO, causal=True, scale=0.35)
    keys = np.arange(N - 8, N)
    rows = np.unique(np.concatenate([[0, 1, 40, 57], keys]))
    g, group = 1, H // Hkv
    sk, sv = np.zeros((N, d)), np.zeros((N, d))
    for h in range(g * group, (g + 1) * group):
        dqs, dks, dvs = oracle.attention_bwd(q[:, h:h + 1, rows], k[:, g:g + 1], v[:, g:g + 1], dO[:, h:h + 1, rows],
                                             causal=True, scale=0.35, q_pos=rows)
        np.testing.assert_allclose(dqs[0, 0], dq[0, h, rows], atol=1e-13)
        sk += dks[0, 0]
        sv += dvs[0, 0]
    np.testing.assert_allclose(sk[keys], dk[0, g, keys], atol=1e-13)
    np.testing.assert_allclose(sv[keys], dv[0, g, keys], atol=1e-13)
    # a key that rows outside the subset also see is not complete
    assert np.abs(sk[10] - dk[0, g, 10]).max() > 1e-6
