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
    "ring_attn_decode_ws_bytes", "ring_attn_decode", "ring_attn_decode_noalloc",
    "ring_attn_bwd_ws_bytes", "ring_attn_bwd", "ring_attn_bwd_share_ws_bytes", "ring_attn_bwd_share",
    "ring_attn_bwd_prep", "ring_attn_bwd_step",
    "ra_last_error", "ra_version", "ra_debug_set_delays", "ra_prof_enable", "ra_prof_reset", "ra_prof_read",
    "ra_diag_mfma_loop", "ra_debug_set_staging",
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
    lib.ring_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, ll, i, i, f, i, vp]
    lib.ring_attn_decode_noalloc.restype = i
    lib.ring_attn_bwd_ws_bytes.argtypes = [i, i, i, ll, i, i, i]
    lib.ring_attn_bwd_ws_bytes.restype = st
    lib.ring_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, ll, i, i, i, i, f, i, vp, vp, st]
    lib.ring_attn_bwd.restype = i
    lib.ring_attn_bwd_share_ws_bytes.argtypes = [i, i, i, ll, i, i, i]
    lib.ring_attn_bwd_share_ws_bytes.restype = st
    lib.ring_attn_bwd_share.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, ll, i, i, i, i, i, f, i, vp,
                                        vp, st]
    lib.ring_attn_bwd_share.restype = i
    lib.ring_attn_bwd_prep.argtypes = [vp, vp, vp, vp, ll, i, i, vp]
    lib.ring_attn_bwd_prep.restype = i
    lib.ring_attn_bwd_step.argtypes = [vp, vp, vp, ra_kv_block, vp, vp, vp, ctypes.POINTER(ra_mask_desc), vp]
    lib.ring_attn_bwd_step.restype = i
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
    lib.ra_debug_set_staging.argtypes = [i]
    lib.ra_debug_set_staging.restype = i
    lib.ra_diag_mfma_loop.argtypes = [i, i, vp, ctypes.POINTER(ctypes.c_double)]
    lib.ra_diag_mfma_loop.restype = i
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


SIZE_MAX = (1 << 64) - 1


def _tensor(t, name, shape=None, dtype=None):
    """Checks a tensor argument's dtype, exact shape and contiguity (raises
    TypeError / ValueError); _devices() then checks where it lives."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _devices(**named):
    """Every tensor must be a device tensor, all on the same device."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _need(t, name):
    _tensor(t, name)
    _devices(**{name: t})


def _workspace(nbytes: int, like, ws=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if ws is not None:
        _tensor(ws, "ws")
        _devices(like=like, ws=ws)
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


def _ws_size(n: int) -> int:
    """A size query's result; SIZE_MAX means the query rejected its arguments."""
    n = int(n)
    if n == SIZE_MAX:
        msg = load().ra_last_error().decode(errors="replace")
        code = RA_ENOMEM if "address space" in msg else RA_EINVAL
        raise RingAttnError(code, msg)
    return n


def ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, dtype_code) -> int:
    return _ws_size(load().ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, dtype_code))


def _qkv(q, k, v):
    """Shapes and dtype of q [B, H, Nq, d] and k, v [B, Hkv, N, d]."""
    _tensor(q, "q")
    code = _dtype_code(q)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D: [B, H, N, d] and [B, Hkv, N, d]")
    B, H, Nq, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    _tensor(k, "k", (B, Hkv, N, d), q.dtype)
    _tensor(v, "v", (B, Hkv, N, d), q.dtype)
    return B, H, Hkv, Nq, N, d, code


def _outputs(q, out, lse, lse_shape):
    torch = _torch()
    if out is not None:
        _tensor(out, "out", tuple(q.shape), q.dtype)
    if lse is not None:
        _tensor(lse, "lse", lse_shape, torch.float32)
    _devices(q=q, out=out, lse=lse)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    return out, lse


def ring_attn_fwd(q, k, v, *, P: int, causal: bool, layout: str = "contiguous", scale: float | None = None,
                  out=None, lse=None, ws=None, stream=None):
    """Full attention by the ring method over P virtual hosts (see ring_attn.h).

    q [B, H, N, d], k, v [B, Hkv, N, d] (bf16 or fp32, contiguous, on the GPU).
    Returns (out [B, H, N, d], lse [B, H, N] fp32).
    """
    lib = load()
    B, H, Hkv, Nq, N, d, code = _qkv(q, k, v)
    if Nq != N:
        raise ValueError("q and k, v must hold the same N tokens")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse, (B, H, N))
    _devices(q=q, k=k, v=v)
    nb = _ws_size(lib.ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, code))
    wst = _workspace(nb, q, ws)
    _check(lib.ring_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, N, d, P,
                             int(bool(causal)), LAYOUTS[layout], scale, code, _stream(stream),
                             _ptr(wst) if wst is not None else None, nb))
    return out, lse


def ring_attn_fwd_share(q, k, v, *, P: int, rank: int, causal: bool, layout: str = "contiguous",
                        scale: float | None = None, out=None, lse=None, ws=None, stream=None):
    """One device's share: q [B, H, N/P, d] of host `rank`; k, v [B, Hkv, N, d]."""
    lib = load()
    B, H, Hkv, Nq, N, d, code = _qkv(q, k, v)
    if Nq * P != N:
        raise ValueError("q must hold N / P rows")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, out, lse, (B, H, Nq))
    _devices(q=q, k=k, v=v)
    nb = _ws_size(lib.ring_attn_fwd_share_ws_bytes(B, H, Hkv, N, d, P, code))
    wst = _workspace(nb, q, ws)
    _check(lib.ring_attn_fwd_share(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, N, d, P,
                                   rank, int(bool(causal)), LAYOUTS[layout], scale, code, _stream(stream),
                                   _ptr(wst) if wst is not None else None, nb))
    return out, lse


def ring_attn_bwd(q, k, v, out, dout, lse, *, P: int, causal: bool, layout: str = "contiguous",
                  scale: float | None = None, dq=None, dk=None, dv=None, ws=None, stream=None):
    """Gradients of ring_attn_fwd by recomputation over a reverse ring.

    q, out, dout [B, H, N, d]; k, v [B, Hkv, N, d] (all bf16 or all fp32);
    lse [B, H, N] fp32 from the forward.  Returns (dq, dk, dv) shaped like
    q, k, v, in their dtype.
    """
    torch = _torch()
    lib = load()
    B, H, Hkv, Nq, N, d, code = _qkv(q, k, v)
    if Nq != N:
        raise ValueError("q and k, v must hold the same N tokens")
    _tensor(out, "out", (B, H, N, d), q.dtype)
    _tensor(dout, "dout", (B, H, N, d), q.dtype)
    _tensor(lse, "lse", (B, H, N), torch.float32)
    for g, like, nm in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if g is not None:
            _tensor(g, nm, tuple(like.shape), like.dtype)
    _devices(q=q, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    nb = _ws_size(lib.ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, code))
    wst = _workspace(nb, q, ws)
    _check(lib.ring_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                             _ptr(dv), B, H, Hkv, N, d, P, int(bool(causal)), LAYOUTS[layout], scale, code,
                             _stream(stream), _ptr(wst) if wst is not None else None, nb))
    return dq, dk, dv


def ring_attn_bwd_share(q, k, v, out, dout, lse, *, P: int, rank: int, causal: bool, layout: str = "contiguous",
                        scale: float | None = None, dq=None, dk=None, dv=None, ws=None, stream=None):
    """One device's share of the backward (see ring_attn.h).

    q, out, dout [B, H, N/P, d] and lse [B, H, N/P] of host `rank` (as
    ring_attn_fwd_share takes and returns them); k, v [B, Hkv, N, d].
    Returns (dq [B, H, N/P, d], dk, dv [B, Hkv, N, d]): the rank's query
    gradient and its contribution to every key's gradient.
    """
    torch = _torch()
    lib = load()
    B, H, Hkv, Nq, N, d, code = _qkv(q, k, v)
    if Nq * P != N:
        raise ValueError("q must hold N / P rows")
    _tensor(out, "out", (B, H, Nq, d), q.dtype)
    _tensor(dout, "dout", (B, H, Nq, d), q.dtype)
    _tensor(lse, "lse", (B, H, Nq), torch.float32)
    for g, like, nm in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if g is not None:
            _tensor(g, nm, tuple(like.shape), like.dtype)
    _devices(q=q, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    nb = _ws_size(lib.ring_attn_bwd_share_ws_bytes(B, H, Hkv, N, d, P, code))
    wst = _workspace(nb, q, ws)
    _check(lib.ring_attn_bwd_share(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                                   _ptr(dk), _ptr(dv), B, H, Hkv, N, d, P, rank, int(bool(causal)),
                                   LAYOUTS[layout], scale, code, _stream(stream),
                                   _ptr(wst) if wst is not None else None, nb))
    return dq, dk, dv


def ring_attn_bwd_prep(out, dout, lse, *, rowstat=None, stream=None):
    """Row statistics of a query block for ring_attn_bwd_step (see ring_attn.h).

    out, dout [B, H, Lq, d] (bf16 or fp32), lse [B, H, Lq] fp32 from the
    forward.  Returns rowstat [B, H, Lq, 2] fp32 (lse * log2 e, dO . O).
    """
    torch = _torch()
    lib = load()
    _tensor(out, "out")
    code = _dtype_code(out)
    if out.dim() != 4:
        raise ValueError("out must be 4-D: [B, H, Lq, d]")
    B, H, Lq, d = out.shape
    _tensor(dout, "dout", tuple(out.shape), out.dtype)
    _tensor(lse, "lse", (B, H, Lq), torch.float32)
    if rowstat is not None:
        _tensor(rowstat, "rowstat", (B, H, Lq, 2), torch.float32)
    _devices(out=out, dout=dout, lse=lse, rowstat=rowstat)
    if rowstat is None:
        rowstat = torch.empty((B, H, Lq, 2), dtype=torch.float32, device=out.device)
    _check(lib.ring_attn_bwd_prep(_ptr(out), _ptr(dout), _ptr(lse), _ptr(rowstat), B * H * Lq, d, code,
                                  _stream(stream)))
    return rowstat


def ring_attn_bwd_step(q_blk, k_blk, v_blk, dout_blk, rowstat, dq_acc, dk_acc, dv_acc, *, causal: bool,
                       layout: str = "contiguous", P: int = 1, q_rank: int = 0, kv_rank: int = 0,
                       scale: float | None = None, stream=None):
    """One (query block, kv block) pair of a ring backward, added in place
    into the fp32 accumulators dq_acc [B, H, Lq, d] and dk_acc, dv_acc
    [B, Hkv, Lkv, d] (see ring_attn.h).  rowstat from ring_attn_bwd_prep."""
    torch = _torch()
    lib = load()
    B, H, Hkv, Lq, Lkv, d, code = _qkv(q_blk, k_blk, v_blk)
    _tensor(dout_blk, "dout_blk", tuple(q_blk.shape), q_blk.dtype)
    _tensor(rowstat, "rowstat", (B, H, Lq, 2), torch.float32)
    _tensor(dq_acc, "dq_acc", (B, H, Lq, d), torch.float32)
    _tensor(dk_acc, "dk_acc", (B, Hkv, Lkv, d), torch.float32)
    _tensor(dv_acc, "dv_acc", (B, Hkv, Lkv, d), torch.float32)
    _devices(q_blk=q_blk, k_blk=k_blk, v_blk=v_blk, dout_blk=dout_blk, rowstat=rowstat, dq_acc=dq_acc,
             dk_acc=dk_acc, dv_acc=dv_acc)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    md = ra_mask_desc(B, H, Hkv, d, Lq, Lkv, scale, code, int(bool(causal)), LAYOUTS[layout], P,
                      q_rank, kv_rank)
    _check(lib.ring_attn_bwd_step(_ptr(q_blk), _ptr(dout_blk), _ptr(rowstat), ra_kv_block(_ptr(k_blk), _ptr(v_blk)),
                                  _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), ctypes.byref(md), _stream(stream)))
    return dq_acc, dk_acc, dv_acc


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
    torch = _torch()
    lib = load()
    B, H, Hkv, Lq, Lkv, d, code = _qkv(q_blk, k_blk, v_blk)
    _tensor(m, "m", (B, H, Lq), torch.float32)
    _tensor(l, "l", (B, H, Lq), torch.float32)
    _tensor(o, "o", (B, H, Lq, d), torch.float32)
    _devices(q_blk=q_blk, k_blk=k_blk, v_blk=v_blk, m=m, l=l, o=o)
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
    _tensor(o, "o", None, torch.float32)
    if o.dim() < 1:
        raise ValueError("o must have a trailing dim axis")
    rows_shape = tuple(o.shape[:-1])
    _tensor(m, "m", rows_shape, torch.float32)
    _tensor(l, "l", rows_shape, torch.float32)
    if out is not None:
        _tensor(out, "out", tuple(o.shape), out_dtype or out.dtype)
    if lse is not None:
        _tensor(lse, "lse", rows_shape, torch.float32)
    _devices(o=o, m=m, l=l, out=out, lse=lse)
    d = o.shape[-1]
    rows = o.numel() // d if d else 0
    if out is None:
        out = torch.empty(o.shape, dtype=out_dtype or torch.bfloat16, device=o.device)
    code = _dtype_code(out)
    if lse is None:
        lse = torch.empty(rows_shape, dtype=torch.float32, device=o.device)
    _check(lib.ring_attn_finalize(_ptr(m), _ptr(l), _ptr(o), _ptr(out), _ptr(lse), rows, d, code,
                                  _stream(stream)))
    return out, lse


def lse_merge(o_a, lse_a, o_b, lse_b, *, stream=None):
    """In-place merge of (o_b, lse_b) into (o_a, lse_a) (fp32)."""
    torch = _torch()
    lib = load()
    _tensor(o_a, "o_a", None, torch.float32)
    if o_a.dim() < 1:
        raise ValueError("o_a must have a trailing dim axis")
    rows_shape = tuple(o_a.shape[:-1])
    _tensor(o_b, "o_b", tuple(o_a.shape), torch.float32)
    _tensor(lse_a, "lse_a", rows_shape, torch.float32)
    _tensor(lse_b, "lse_b", rows_shape, torch.float32)
    _devices(o_a=o_a, o_b=o_b, lse_a=lse_a, lse_b=lse_b)
    d = o_a.shape[-1]
    rows = o_a.numel() // d if d else 0
    _check(lib.lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), rows, d, _stream(stream)))
    return o_a, lse_a


def ring_attn_decode_ws_bytes(B, H, Hkv, L, d, P) -> int:
    return _ws_size(load().ring_attn_decode_ws_bytes(B, H, Hkv, L, d, P))


def _decode_args(q, k, v, out, lse):
    B, H, Hkv, one, L, d, code = _qkv(q, k, v)
    if one != 1:
        raise ValueError("q must be [B, H, 1, d]")
    out, lse = _outputs(q, out, lse, (B, H))
    _devices(q=q, k=k, v=v)
    return B, H, Hkv, L, d, code, out, lse


def ring_attn_decode(q, k, v, *, P: int, scale: float | None = None, out=None, lse=None, ws=None,
                     stream=None):
    """Split-KV decode: q [B, H, 1, d]; k, v [B, Hkv, L, d] (all bf16 or all
    fp32) -> (out [B, H, 1, d] in their dtype, lse [B, H] fp32)."""
    lib = load()
    B, H, Hkv, L, d, code, out, lse = _decode_args(q, k, v, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nb = ring_attn_decode_ws_bytes(B, H, Hkv, L, d, P)
    wst = _workspace(nb, q, ws)
    _check(lib.ring_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, L, d, P, scale,
                                code, _stream(stream), _ptr(wst) if wst is not None else None, nb))
    return out, lse


def ring_attn_decode_noalloc(q, k, v, *, P: int, scale: float | None = None, out=None, lse=None, stream=None):
    """ring_attn_decode with the library's static scratch instead of a
    workspace (no device allocation inside the call when out and lse are
    given)."""
    lib = load()
    B, H, Hkv, L, d, code, out, lse = _decode_args(q, k, v, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.ring_attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Hkv, L, d, P, scale,
                                        code, _stream(stream)))
    return out, lse


def debug_set_delays(compute_us: int = 0, copy_us: int = 0) -> None:
    """Test hook: bounded spins before every step kernel / staging copy."""
    _check(load().ra_debug_set_delays(int(compute_us), int(copy_us)))


def diag_mfma_loop(workgroups: int, iters: int, stream=None) -> float:
    """Counter calibration: a register-only bf16 MFMA loop; returns its MFMA count."""
    n = ctypes.c_double()
    _check(load().ra_diag_mfma_loop(int(workgroups), int(iters), _stream(stream), ctypes.byref(n)))
    return n.value


def debug_set_staging(on: bool = True) -> None:
    """Test / measurement hook: ring steps read their kv blocks in place (off) or staged (on, default)."""
    _check(load().ra_debug_set_staging(int(bool(on))))


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
