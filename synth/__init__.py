"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic. It only draws i.i.d. N(0, 1)
values and rounds them to the storage precision, so that both sides of a
parity check see bit-identical inputs.

Recipe (one generator per [N, d] slab, so any slab can be regenerated alone):
    rng  = numpy.random.default_rng([seed, tensor_id, b, h])
    x    = rng.standard_normal((N, d), dtype=float32)
    bf16 = round-to-nearest-even of the float32 bit pattern to its top 16 bits
tensor_id: q = 0, k = 1, v = 2.  The seed is the workload's own number.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
TENSOR_DOUT = 3   # upstream gradient of the output (backward tests)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite normals, so no NaN/inf special case is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the float32 values they encode (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def slab(seed: int, tensor_id: int, b: int, h: int, n: int, d: int) -> np.ndarray:
    """One [n, d] float32 slab of N(0, 1) draws (before any rounding)."""
    rng = np.random.default_rng([int(seed), int(tensor_id), int(b), int(h)])
    return rng.standard_normal((n, d), dtype=np.float32)


def slab_bits(seed: int, tensor_id: int, b: int, h: int, n: int, d: int) -> np.ndarray:
    """One [n, d] slab as bf16 bit patterns (uint16)."""
    return bf16_bits(slab(seed, tensor_id, b, h, n, d))


def tensor(seed: int, tensor_id: int, B: int, H: int, n: int, d: int, dtype: str,
           threads: int | None = None) -> np.ndarray:
    """A [B, H, n, d] tensor.

    dtype "f32": float32 values.  dtype "bf16": uint16 bf16 bit patterns.
    Slabs are generated in parallel; each slab's values do not depend on
    how many threads ran.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    out = np.empty((B, H, n, d), dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        x = slab(seed, tensor_id, b, h, n, d)
        out[b, h] = x if dtype == "f32" else bf16_bits(x)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def uniform_tensor(seed: int, tensor_id: int, B: int, H: int, n: int, d: int, lo: float, hi: float,
                   dtype: str) -> np.ndarray:
    """A [B, H, n, d] tensor of U(lo, hi) draws, in storage form like `tensor`.

    Used for values of one sign and large magnitude (rows whose output is
    far from zero)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    out = np.empty((B, H, n, d), dtype=np.float32 if dtype == "f32" else np.uint16)
    for b in range(B):
        for h in range(H):
            rng = np.random.default_rng([int(seed), int(tensor_id), int(b), int(h), 1])
            x = rng.uniform(lo, hi, (n, d)).astype(np.float32)
            out[b, h] = x if dtype == "f32" else bf16_bits(x)
    return out


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of a tensor made by `tensor` as float32 (exact for bf16)."""
    return x if dtype == "f32" else bf16_bits_to_f32(x)


def qkv(seed: int, B: int, H: int, Hkv: int, N: int, d: int, dtype: str,
        Nq: int | None = None, threads: int | None = None):
    """(q, k, v) with q [B, H, Nq, d] and k, v [B, Hkv, N, d].

    Nq defaults to N.  Returned in storage form (float32, or uint16 bf16 bits).
    """
    nq = N if Nq is None else Nq
    q = tensor(seed, TENSOR_Q, B, H, nq, d, dtype, threads)
    k = tensor(seed, TENSOR_K, B, Hkv, N, d, dtype, threads)
    v = tensor(seed, TENSOR_V, B, Hkv, N, d, dtype, threads)
    return q, k, v
