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
