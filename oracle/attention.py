"""fp64 CPU oracle: plain materialized attention, written from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP product path
never imports or runs this file.

Pages cited (by title; section or equation named alone):
  [TKG]  "RingAttention 심층 아키텍처: 통신-연산 완전 중첩과 블록 단위 온라인
         소프트맥스로 1,000만 토큰 컨텍스트를 정복한 분산 어텐션 엔지니어링"
         (techknowgenie.com).  §1 (materialized N x N score matrix),
         §3 (blockwise online-softmax derivation: S, m_block, m_new,
         alpha/beta, P_curr/l_curr/l_new, O_new, O_final), §7 (causal mask,
         striped round-robin sharding).
  [AIT]  FlashAttention video summary (aitrends.kr), chapter "Attention 연산의
         기본 과정" (scores, max-subtracted softmax, weighted sum of V).

The ring method claims to reach full attention exactly ([TKG] §3 closing
paragraph, §8), so this oracle is that plain definition, evaluated in fp64
per chunk of query rows:

    S_ij  = scale * <q_i, k_j>                     [TKG] §3, equation for S
    valid = not causal  or  pos_k(j) <= pos_q(i)   [TKG] §7 (past tokens only;
                                                   a token sees itself)
    m_i   = max_{valid j} S_ij                     [AIT] max-subtracted softmax
    w_ij  = exp(S_ij - m_i) on valid j, else 0
    l_i   = sum_j w_ij
    O_i   = sum_j w_ij v_j / l_i                   [TKG] §3, O_final = O / l
    lse_i = m_i + ln l_i        (natural log of scaled logits; the pages keep
                                 only (m, l); lse is their combination)

A query row with no valid key has O = 0 and lse = -inf.
GQA: query head h reads kv head floor(h * Hkv / H) (consecutive groups).

Readings where the pages are silent are listed with the repository's design
notes; each function below names the one it uses.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # keep BLAS single-threaded inside our own thread pool
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None

_CHUNK_ELEMS = 1 << 24  # score elements materialized per work unit (128 MiB fp64)


def _threads(threads):
    if threads:
        return int(threads)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def host_positions(N: int, P: int, layout: str) -> list[np.ndarray]:
    """Global token positions owned by each of the P hosts.

    [TKG] §2: each host holds B = N / P tokens.  "contiguous": host r holds
    tokens r*B .. r*B + B - 1.  "striped" ([TKG] §7, round-robin): host r
    holds tokens r, r + P, r + 2P, ...  "zigzag" ([CML] "İddia ve Gerçeklik"
    names zigzag schedules beside striped ones; the pages give no formula,
    so this is the plain reading): the sequence is cut into 2P equal chunks
    and host r holds chunk r followed by chunk 2P-1-r, pairing an early
    chunk with a late one.
    """
    if N % P:
        raise ValueError("N must be a multiple of P")
    Bl = N // P
    if layout == "contiguous":
        return [np.arange(r * Bl, (r + 1) * Bl, dtype=np.int64) for r in range(P)]
    if layout == "striped":
        return [np.arange(r, N, P, dtype=np.int64) for r in range(P)]
    if layout == "zigzag":
        if N % (2 * P):
            raise ValueError("zigzag needs N to be a multiple of 2P")
        C = N // (2 * P)
        return [np.concatenate([np.arange(r * C, (r + 1) * C, dtype=np.int64),
                                np.arange((2 * P - 1 - r) * C, (2 * P - r) * C, dtype=np.int64)])
                for r in range(P)]
    raise ValueError(f"unknown layout {layout!r}")


def attention_rows(q_rows, k, v, *, scale, causal, q_pos=None, k_pos=None):
    """Plain attention for some query rows against one key/value head.

    q_rows [R, d], k [Nk, d], v [Nk, dv]; positions are int arrays (default:
    natural order).  Returns (O [R, dv], lse [R], m [R], l [R]) in fp64, where
    (m, l) are the row max of the valid scaled scores and the sum of
    exp(S - m) over valid keys.
    """
    q = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(k, dtype=np.float64)
    V = np.asarray(v, dtype=np.float64)
    R, Nk = q.shape[0], K.shape[0]
    S = (q @ K.T) * float(scale)                                  # [R, Nk]
    if causal:
        qp = np.arange(R, dtype=np.int64) if q_pos is None else np.asarray(q_pos, np.int64)
        kp = np.arange(Nk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, np.int64)
        valid = kp[None, :] <= qp[:, None]
    else:
        valid = np.ones((R, Nk), dtype=bool)
    S = np.where(valid, S, -np.inf)
    any_valid = valid.any(axis=1)
    m = np.where(any_valid, S.max(axis=1, initial=-np.inf), -np.inf)
    m_safe = np.where(any_valid, m, 0.0)
    w = np.where(valid, np.exp(S - m_safe[:, None]), 0.0)
    l = w.sum(axis=1)
    num = w @ V
    l_safe = np.where(any_valid, l, 1.0)
    O = np.where(any_valid[:, None], num / l_safe[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(any_valid, m_safe + np.log(l_safe), -np.inf)
    return O, lse, m, l


def attention(q, k, v, *, scale=None, causal=False, q_pos=None, k_pos=None,
              rows=None, heads=None, threads=None):
    """Full attention O, lse for q [B, H, Nq, d], k, v [B, Hkv, Nk, d].

    q_pos / k_pos: global positions of the query / key rows (default: their
    index).  rows: optional query-row indices to evaluate (a sample); the
    result then has len(rows) rows.  heads: optional list of (b, h) pairs to
    evaluate; others are left as NaN.  Returns fp64 (O, lse).
    """
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch between q, k, v")
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    dv = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    row_idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    qp_all = np.arange(Nq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, np.int64)
    kp = np.arange(Nk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, np.int64)
    R = row_idx.shape[0]
    O = np.full((B, H, R, dv), np.nan)
    lse = np.full((B, H, R), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    chunk = max(1, min(R, _CHUNK_ELEMS // max(1, Nk)))
    group = H // Hkv
    # one kv plane at a time, converted to fp64 once and shared by its units
    planes = {}
    for (b, h) in pairs:
        planes.setdefault((b, h // group), []).append(h)
    nthr = _threads(threads)

    def run_plane(b, g, hs):
        K = np.asarray(k[b, g], dtype=np.float64)
        V = np.asarray(v[b, g], dtype=np.float64)
        units = [(h, s) for h in hs for s in range(0, R, chunk)]

        def work(unit):
            h, s = unit
            sel = row_idx[s:s + chunk]
            o, ls, _, _ = attention_rows(q[b, h, sel], K, V, scale=scale,
                                         causal=causal, q_pos=qp_all[sel], k_pos=kp)
            O[b, h, s:s + chunk] = o
            lse[b, h, s:s + chunk] = ls

        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(work, units))

    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            for (b, g), hs in planes.items():
                run_plane(b, g, hs)
    else:  # pragma: no cover
        for (b, g), hs in planes.items():
            run_plane(b, g, hs)
    return O, lse


def decode(q, k, v, *, scale=None, threads=None):
    """Split-KV decode target: one query token per sequence, no mask.

    q [B, H, 1, d]; k, v [B, Hkv, L, d].  Reading (pages silent on the decode
    query's position): the new token sees every cached key, which is the last
    row of a causal prefill whose final query is q.
    """
    return attention(q, k, v, scale=scale, causal=False, threads=threads)


def step_partial(q_blk, k_blk, v_blk, *, scale, causal, q_pos=None, k_pos=None):
    """One ring step's contribution for one (query block, kv block) pair.

    [TKG] §3: S_ik, m_block = rowmax(S_ik), P_curr = exp(S_ik - m_block),
    l_curr = rowsum(P_curr), and the block's P_curr V_k.  q_blk [R, d],
    k_blk / v_blk [Nk, d].  Returns (m, l, o_unnormalized, lse, O_normalized)
    in fp64.  Rows with no valid key: m = -inf, l = 0, o = 0, lse = -inf.
    """
    O, lse, m, l = attention_rows(q_blk, k_blk, v_blk, scale=scale, causal=causal,
                                  q_pos=q_pos, k_pos=k_pos)
    o_un = O * l[:, None]
    return m, l, o_un, lse, O


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two normalized partial results over disjoint key sets.

    Not written out on the pages; it is what the [TKG] §3 m_new / alpha /
    beta / l_new / O_new updates do when two partial states meet, expressed
    with lse = m + ln l:  lse = ln(e^lse_a + e^lse_b),
    O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.  Both -inf gives O = 0,
    lse = -inf.  Shapes: o [..., d], lse [...]; returns fp64 (O, lse).
    """
    a = np.asarray(lse_a, dtype=np.float64)
    b = np.asarray(lse_b, dtype=np.float64)
    Oa = np.asarray(o_a, dtype=np.float64)
    Ob = np.asarray(o_b, dtype=np.float64)
    M = np.maximum(a, b)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    wa = np.where(np.isfinite(a), np.exp(a - Ms), 0.0)
    wb = np.where(np.isfinite(b), np.exp(b - Ms), 0.0)
    tot = wa + wb
    tot_s = np.where(finite, tot, 1.0)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, Ms + np.log(tot_s), -np.inf)
    O = np.where(finite[..., None],
                 (wa[..., None] * Oa + wb[..., None] * Ob) / tot_s[..., None], 0.0)
    return O, lse


def pair_counts(N: int, P: int, layout: str, causal: bool) -> np.ndarray:
    """Unmasked (query, key) pairs for each (query host, kv host) block.

    Used for the causal-adjusted FLOP count (4 d per unmasked pair per query
    head, [TKG] §4 table: 4 B^2 d per block pair) and for the striped
    balance check ([TKG] §7).  Exact integer counts via positions.
    """
    pos = host_positions(N, P, layout)
    out = np.zeros((P, P), dtype=np.int64)
    for rq in range(P):
        qp = np.sort(pos[rq])
        for rk in range(P):
            kp = np.sort(pos[rk])
            if causal:
                out[rq, rk] = int(np.searchsorted(kp, qp, side="right").sum())
            else:
                out[rq, rk] = qp.size * kp.size
    return out
