"""Helpers shared by the tests: seeded inputs on the device and comparisons.

Inputs come from the `synth` generator (no attention arithmetic); expected
values come only from `oracle`.
"""
from __future__ import annotations

import numpy as np

import synth

# Tolerances (max absolute error against the fp64 oracle on the same
# rounded inputs): fp32 path 1e-5 on O and lse; bf16 path 1e-2 on O and
# 1e-3 on lse.
TOL = {"f32": (1e-5, 1e-5), "bf16": (1e-2, 1e-3)}


def to_dev(x: np.ndarray, dtype: str, device="cuda:0"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def from_dev(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().float().cpu().numpy()


def host_vals(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values of a synth tensor (exact for bf16 storage)."""
    return synth.as_f32(x, dtype)


def max_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(d)) if d.size else 0.0


def assert_close(got_o, got_lse, want_o, want_lse, dtype: str, what: str = ""):
    to, tl = TOL[dtype]
    eo = max_err(got_o, want_o)
    el = max_err(got_lse, want_lse)
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite output"
    assert eo <= to and el <= tl, f"{what}: max|dO|={eo:.3e} (tol {to}) max|dlse|={el:.3e} (tol {tl})"
    return eo, el


def sample_rows(N: int, P: int, layout: str, n_random: int, seed: int, tile: int = 128) -> np.ndarray:
    """Row sample: first/last row of every host block (in each layout's host
    order), rows around every `tile` boundary of a host block, plus random rows."""
    Bl = N // P
    rows = set()
    for r in range(P):
        for i in (0, 1, Bl - 2, Bl - 1):
            if 0 <= i < Bl:
                rows.add(r * Bl + i if layout == "contiguous" else i * P + r)
    for t in range(0, Bl, tile * max(1, Bl // tile // 16)):
        for i in (t - 1, t, t + 1):
            if 0 <= i < Bl:
                for r in (0, P - 1):
                    rows.add(r * Bl + i if layout == "contiguous" else i * P + r)
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, N, n_random))
    return np.array(sorted(rows), dtype=np.int64)
