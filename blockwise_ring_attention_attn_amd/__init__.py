"""MI355X (gfx950) blockwise ring attention: thin Python binding.

Every function here marshals arguments to the C ABI of include/ring_attn.h
(same names) and returns the tensors the library wrote.  All arithmetic runs
in the HIP kernels of libringattn.so; PyTorch only provides device memory
and the current stream.  If the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libringattn.so")

RA_OK, RA_EINVAL, RA_ENOMEM, RA_EHIP, RA_EUNSUPPORTED = 0, 1, 2, 3, 4
RA_CONTIGUOUS, RA_STRIPED, RA_ZIGZAG = 0, 1, 2
RA_F32, RA_BF16 = 0, 1
LAYOUTS = {"contiguous": RA_CONTIGUOUS, "striped": RA_STRIPED, "zigzag": RA_ZIGZAG}

# Every symbol declared in include/ring_attn.h.
EXPORTS = (
    "ring_attn_fwd_ws_bytes", "ring_attn_fwd",
    "ring_attn_fwd_share_ws_bytes", "ring_attn_fwd_share",
    "ring_attn_step", "ring_attn_finalize", "lse_merge",
    "ring_attn_decode_ws_bytes", "ring_attn_decode",
    "ring_attn_bwd_ws_bytes", "ring_attn_bwd",
    "ra_last_error", "ra_version", "ra_debug_set_delays", "ra_prof_enable", "ra_prof_reset", "ra_prof_read",
)


class RingAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ring_attn status {status}: {msg}")
        self.status = status


class ra_kv_block(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class ra_mask_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int),
                ("Lq", ctypes.c_longlong), ("Lkv", ctypes.c_longlong), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int), ("causal", ctypes.c_int), ("layout", ctypes.c_int),
                ("P", ctypes.c_int), ("q_rank", ctypes.c_int), ("kv_rank", ctypes.c_int)]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libringattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"HIP library not built: {p} is missing "
                           "(run python -m blockwise_ring_attention_attn_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i, ll, f, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_size_t
    lib.ring_attn_fwd_ws_bytes.argtypes = [i, i, i, ll, i, i, i]
    lib.ring_attn_fwd_ws_bytes.restype = st
    lib.ring_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, ll, i, i, i, i, f, i, vp, vp, st]
    lib.ring_attn_fwd.restype = i
    lib.ring_attn_fwd_share_ws_bytes.argtypes = [i, i, i, ll, i, i, i]
    lib.ring_attn_fwd_share_ws_bytes.restype = st
    lib.ring_attn_fwd_share.argtypes = [vp, vp, vp, vp, vp, i, i, i, ll, i, i, i, i, i, f, i, vp, vp, st]
    lib.ring_attn_fwd_share.restype = i
    lib.ring_attn_step.argtypes = [vp, ra_kv_block, vp, vp, vp, ctypes.POINTER(ra_mask_desc), vp]
    lib.ring_attn_step.restype = i
    lib.ring_attn_finalize.argtypes = [vp, vp, vp, vp, vp, ll, i, i, vp]
    lib.ring_attn_finalize.restype = i
    lib.lse_merge.argtypes = [vp, vp, vp, vp, ll, i, vp]
    lib.lse_merge.restype = i
    lib.ring_attn_decode_ws_bytes.argtypes = [i, i, i, ll, i, i]
    lib.ring_attn_decode_ws_bytes.restype = st
    lib.ring_attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, ll, i, i, f, i, vp, vp, st]
    lib.ring_attn_decode.restype = i
    lib.ring_attn_bwd_ws_bytes.argtypes = [i, i, i, ll, i, i, i]
    lib.ring_attn_bwd_ws_bytes.restype = st
    lib.ring_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, ll, i, i, i, i, f, i, vp, vp, st]
    lib.ring_attn_bwd.restype = i
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_version.argtypes = []
    lib.ra_version.restype = ctypes.c_char_p
    lib.ra_debug_set_delays.argtypes = [i, i]
    lib.ra_debug_set_delays.restype = i
    lib.ra_prof_enable.argtypes = [i]
    lib.ra_prof_enable.restype = i
    lib.ra_prof_reset.argtypes = []
    lib.ra_prof_reset.restype = i
    lib.ra_prof_read.argtypes = [ctypes.POINTER(ctypes.c_double)]
    lib.ra_prof_read.restype = i
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != RA_OK:
        msg = load().ra_last_error().decode(errors="replace")
        raise RingAttnError(status, msg)


def _torch():
    import torch  # plumbing only: device memory and streams
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> int:
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device, ws=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, dtype_code) -> int:
    return int(load().ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, dtype_code))


def ring_attn_fwd(q, k, v, *, P: int, causal: bool, layout: str = "contiguous", scale: float | None = None,
                  out=None, lse=None, ws=None, stream=None):
    """Full attention by the ring method over P virtual hosts (see ring_attn.h).

    q [B, H, N, d], k, v [B, Hkv, N, d] (bf16 or fp32, contiguous, on the GPU).
    Returns (out [B, H, N, d], lse [B, H, N] fp32).
    """
    torch = _torch()
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    code = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k, v must be [B, Hkv, N, d]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    nb = lib.ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, code)
    wst = _workspace(nb, q.device, ws)
    _check(lib.ring_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, N, d, P,
                             int(bool(causal)), LAYOUTS[layout], scale, code, _stream(stream),
                             _ptr(wst) if wst is not None else None, nb))
    return out, lse


def ring_attn_fwd_share(q, k, v, *, P: int, rank: int, causal: bool, layout: str = "contiguous",
                        scale: float | None = None, out=None, lse=None, ws=None, stream=None):
    """One device's share: q [B, H, N/P, d] of host `rank`; k, v [B, Hkv, N, d]."""
    torch = _torch()
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, H, Nq, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    code = _dtype_code(q)
    if Nq * P != N:
        raise ValueError("q must hold N / P rows")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    nb = lib.ring_attn_fwd_share_ws_bytes(B, H, Hkv, N, d, P, code)
    wst = _workspace(nb, q.device, ws)
    _check(lib.ring_attn_fwd_share(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, N, d, P,
                                   rank, int(bool(causal)), LAYOUTS[layout], scale, code, _stream(stream),
                                   _ptr(wst) if wst is not None else None, nb))
    return out, lse


def ring_attn_bwd(q, k, v, out, dout, lse, *, P: int, causal: bool, layout: str = "contiguous",
                  scale: float | None = None, dq=None, dk=None, dv=None, ws=None, stream=None):
    """Gradients of ring_attn_fwd by recomputation over a reverse ring.

    q, out, dout [B, H, N, d]; k, v [B, Hkv, N, d] (bf16); lse [B, H, N] fp32
    from the forward.  Returns (dq, dk, dv) shaped like q, k, v.
    """
    torch = _torch()
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"), (lse, "lse")):
        _need(t, n)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    code = _dtype_code(q)
    if any(t.dtype != q.dtype for t in (k, v, out, dout)):
        raise TypeError("q, k, v, out, dout must share a dtype")
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, d):
        raise ValueError("k, v must be [B, Hkv, N, d]")
    if tuple(out.shape) != (B, H, N, d) or tuple(dout.shape) != (B, H, N, d) or tuple(lse.shape) != (B, H, N):
        raise ValueError("out, dout must be [B, H, N, d] and lse [B, H, N]")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    nb = lib.ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, code)
    wst = _workspace(nb, q.device, ws)
    _check(lib.ring_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                             _ptr(dv), B, H, Hkv, N, d, P, int(bool(causal)), LAYOUTS[layout], scale, code,
                             _stream(stream), _ptr(wst) if wst is not None else None, nb))
    return dq, dk, dv


def init_state(B, H, Lq, d, device):
    """Fresh online-softmax state (m = -inf, l = 0, o = 0) for ring_attn_step."""
    torch = _torch()
    m = torch.full((B, H, Lq), float("-inf"), dtype=torch.float32, device=device)
    l = torch.zeros((B, H, Lq), dtype=torch.float32, device=device)
    o = torch.zeros((B, H, Lq, d), dtype=torch.float32, device=device)
    return m, l, o


def ring_attn_step(q_blk, k_blk, v_blk, m, l, o, *, causal: bool, layout: str = "contiguous", P: int = 1,
                   q_rank: int = 0, kv_rank: int = 0, scale: float | None = None, stream=None):
    """One ring step updating (m, l, o) in place (see ring_attn.h)."""
    lib = load()
    for t, n in ((q_blk, "q_blk"), (k_blk, "k_blk"), (v_blk, "v_blk"), (m, "m"), (l, "l"), (o, "o")):
        _need(t, n)
    B, H, Lq, d = q_blk.shape
    Hkv, Lkv = k_blk.shape[1], k_blk.shape[2]
    code = _dtype_code(q_blk)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    md = ra_mask_desc(B, H, Hkv, d, Lq, Lkv, scale, code, int(bool(causal)), LAYOUTS[layout], P,
                      q_rank, kv_rank)
    _check(lib.ring_attn_step(_ptr(q_blk), ra_kv_block(_ptr(k_blk), _ptr(v_blk)), _ptr(m), _ptr(l), _ptr(o),
                              ctypes.byref(md), _stream(stream)))
    return m, l, o


def ring_attn_finalize(m, l, o, *, out_dtype=None, out=None, lse=None, stream=None):
    """(out, lse) = (o / l, m + ln l) for the rows of the state."""
    torch = _torch()
    lib = load()
    d = o.shape[-1]
    rows = o.numel() // d
    out_dtype = out_dtype or torch.bfloat16
    out = torch.empty(o.shape, dtype=out_dtype, device=o.device) if out is None else out
    lse = torch.empty(m.shape, dtype=torch.float32, device=o.device) if lse is None else lse
    _check(lib.ring_attn_finalize(_ptr(m), _ptr(l), _ptr(o), _ptr(out), _ptr(lse), rows, d,
                                  _dtype_code(out), _stream(stream)))
    return out, lse


def lse_merge(o_a, lse_a, o_b, lse_b, *, stream=None):
    """In-place merge of (o_b, lse_b) into (o_a, lse_a) (fp32)."""
    lib = load()
    for t, n in ((o_a, "o_a"), (lse_a, "lse_a"), (o_b, "o_b"), (lse_b, "lse_b")):
        _need(t, n)
    d = o_a.shape[-1]
    rows = o_a.numel() // d
    _check(lib.lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), rows, d, _stream(stream)))
    return o_a, lse_a


def ring_attn_decode(q, k, v, *, P: int, scale: float | None = None, out=None, lse=None, ws=None,
                     stream=None):
    """Split-KV decode: q [B, H, 1, d]; k, v [B, Hkv, L, d] -> (out [B, H, 1, d], lse [B, H])."""
    torch = _torch()
    lib = load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    B, H, one, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    if one != 1:
        raise ValueError("q must be [B, H, 1, d]")
    code = _dtype_code(q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if lse is None else lse
    nb = lib.ring_attn_decode_ws_bytes(B, H, Hkv, L, d, P)
    wst = _workspace(nb, q.device, ws)
    _check(lib.ring_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, L, d, P, scale,
                                code, _stream(stream), _ptr(wst) if wst is not None else None, nb))
    return out, lse


def debug_set_delays(compute_us: int = 0, copy_us: int = 0) -> None:
    """Test hook: bounded spins before every step kernel / staging copy."""
    _check(load().ra_debug_set_delays(int(compute_us), int(copy_us)))


def prof_enable(on: bool = True) -> None:
    _check(load().ra_prof_enable(int(bool(on))))


def prof_reset() -> None:
    _check(load().ra_prof_reset())


def prof_read() -> dict:
    """Event-timed totals of the fused step and decode kernels since prof_reset()."""
    buf = (ctypes.c_double * 6)()
    _check(load().ra_prof_read(buf))
    return {"step_ms": buf[0], "step_launches": int(buf[1]), "decode_ms": buf[2],
            "decode_launches": int(buf[3]), "step_flops": buf[4], "decode_bytes": buf[5]}
