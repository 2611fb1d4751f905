"""fp64 CPU oracle for the attention backward pass (gradients of the plain
definition).

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP product path
never imports or runs this file.

Pages cited (by title; section named alone):
  [TKG]  "RingAttention 심층 아키텍처: 통신-연산 완전 중첩과 블록 단위 온라인
         소프트맥스로 1,000만 토큰 컨텍스트를 정복한 분산 어텐션 엔지니어링"
         (techknowgenie.com).  §7, "활성화 체크포인팅과 메모리 재연산": the
         backward pass keeps only each block's queries and the row statistics
         (m, l), sends the key/value blocks around the ring the other way and
         recomputes the attention map where it is needed.

The pages do not write the gradient formulas out; what the ring recomputes
is the derivative of the forward definition (see attention.py):

    S = scale * Q K^T (masked entries -inf),  P = softmax_rows(S),  O = P V

For a loss with upstream gradient dO = dL/dO, the chain rule gives

    dV = P^T dO                      (O is linear in V)
    dP = dO V^T
    D_i = sum_j P_ij dP_ij  (= dO_i . O_i)
    dS = P * (dP - D[:, None])       (Jacobian of a row softmax)
    dQ = scale * dS K,   dK = scale * dS^T Q

Masked entries have P = 0, hence dS = 0.  A query row with no visible key
has P = 0 and contributes nothing.  With grouped-query attention, dK and dV
of kv head g sum the contributions of all query heads that read it.  This
module evaluates those formulas directly in fp64, one (batch, head) at a
time, with the full score matrix materialized (small and moderate sizes).
"""
from __future__ import annotations

import math

import numpy as np


def _probs(q, k, *, scale, causal, q_pos, k_pos):
    """Row-softmax P of the masked scaled scores, fp64 [Nq, Nk]."""
    S = (q @ k.T) * float(scale)
    Nq, Nk = S.shape
    if causal:
        qp = np.arange(Nq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, np.int64)
        kp = np.arange(Nk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, np.int64)
        valid = kp[None, :] <= qp[:, None]
    else:
        valid = np.ones((Nq, Nk), dtype=bool)
    any_valid = valid.any(axis=1)
    S = np.where(valid, S, -np.inf)
    m = np.where(any_valid, S.max(axis=1, initial=-np.inf), 0.0)
    w = np.where(valid, np.exp(S - m[:, None]), 0.0)
    l = w.sum(axis=1)
    return w / np.where(any_valid, l, 1.0)[:, None]


def attention_bwd(q, k, v, dout, *, scale=None, causal=False, q_pos=None, k_pos=None, parts=False):
    """Gradients (dq, dk, dv) of the plain attention definition, fp64.

    q, dout [B, H, Nq, d]; k, v [B, Hkv, Nk, d]; query head h reads kv head
    floor(h * Hkv / H).  q_pos / k_pos: global positions (default: the row
    index).  With parts=True also returns a dict of the per-(b, h) fp64
    matrices P, dS and the vectors D (for error bounds in tests).
    """
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    group = H // Hkv
    dq = np.zeros((B, H, Nq, d))
    dk = np.zeros((B, Hkv, Nk, d))
    dv = np.zeros((B, Hkv, Nk, v.shape[3]))
    saved = {}
    for b in range(B):
        for h in range(H):
            g = h // group
            Q = np.asarray(q[b, h], dtype=np.float64)
            K = np.asarray(k[b, g], dtype=np.float64)
            V = np.asarray(v[b, g], dtype=np.float64)
            dO = np.asarray(dout[b, h], dtype=np.float64)
            P = _probs(Q, K, scale=scale, causal=causal, q_pos=q_pos, k_pos=k_pos)
            dP = dO @ V.T
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            dq[b, h] = scale * (dS @ K)
            dk[b, g] += scale * (dS.T @ Q)
            dv[b, g] += P.T @ dO
            if parts:
                saved[(b, h)] = {"P": P, "dS": dS, "D": D}
    if parts:
        return dq, dk, dv, saved
    return dq, dk, dv


def attention_bwd_sampled(q, k, v, dout, *, b, h, rows, keys, scale=None, causal=False, chunk=1024):
    """Gradients of one (batch b, query head h) at sampled positions, fp64.

    Returns (dq_rows, dk_keys, dv_keys, parts): dq of the sampled query rows,
    and this head's contribution to dk, dv of the sampled key rows of its kv
    head g = h * Hkv // H (with grouped heads the full dk, dv of kv head g sum
    the contributions of its H / Hkv query heads; with H == Hkv this is the
    whole gradient).  Positions are the row indices (natural token order).

    The formulas are those of `attention_bwd`, evaluated without the full
    [N, N] matrices: a first pass over chunks of query rows forms each row's
    lse, O and delta = dO . O (and the sampled rows' P, dS); a second pass
    forms the sampled keys' columns of P and dS from the stored lse and delta.
    `parts` holds, for error bounds: P and dS of the sampled rows (all keys),
    P and dS of the sampled keys' columns (all rows), delta, O of all rows, and
    od_i = sum_c |dO_ic| (|O_ic| + sum_j P_ij |v_jc|).
    """
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    if Nk != N:
        raise ValueError("the sampled form takes self-attention shapes (Nk == Nq)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    g = h // (H // Hkv)
    Q = np.asarray(q[b, h], dtype=np.float64)
    K = np.asarray(k[b, g], dtype=np.float64)
    V = np.asarray(v[b, g], dtype=np.float64)
    dO = np.asarray(dout[b, h], dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    absV = np.abs(V)
    lse = np.empty(N)
    delta = np.empty(N)
    od = np.empty(N)
    O = np.empty((N, V.shape[1]))
    P_rows = np.zeros((len(rows), N))
    dS_rows = np.zeros((len(rows), N))
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        nk = r1 if causal else N                      # keys any row of the chunk can see
        S = (Q[r0:r1] @ K[:nk].T) * float(scale)
        if causal:
            S = np.where(np.arange(nk)[None, :] <= np.arange(r0, r1)[:, None], S, -np.inf)
        m = S.max(axis=1)
        Pc = np.exp(S - m[:, None])
        lc = Pc.sum(axis=1)
        Pc /= lc[:, None]
        lse[r0:r1] = m + np.log(lc)
        O[r0:r1] = Pc @ V[:nk]
        delta[r0:r1] = (dO[r0:r1] * O[r0:r1]).sum(axis=1)
        od[r0:r1] = (np.abs(dO[r0:r1]) * (np.abs(O[r0:r1]) + Pc @ absV[:nk])).sum(axis=1)
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        if sel.size:
            Pr = Pc[rows[sel] - r0]
            dPr = dO[rows[sel]] @ V[:nk].T
            P_rows[sel, :nk] = Pr
            dS_rows[sel, :nk] = Pr * (dPr - delta[rows[sel]][:, None])
    dq_rows = float(scale) * (dS_rows @ K)
    Sk = (Q @ K[keys].T) * float(scale)                      # [N, len(keys)]
    if causal:
        Sk = np.where(keys[None, :] <= np.arange(N)[:, None], Sk, -np.inf)
    P_keys = np.exp(Sk - lse[:, None])
    dS_keys = P_keys * (dO @ V[keys].T - delta[:, None])
    dv_keys = P_keys.T @ dO
    dk_keys = float(scale) * (dS_keys.T @ Q)
    parts = {"P_rows": P_rows, "dS_rows": dS_rows, "P_keys": P_keys, "dS_keys": dS_keys,
             "delta": delta, "O": O, "od": od, "lse": lse}
    return dq_rows, dk_keys, dv_keys, parts
