"""Host-only checks of the C ABI (no GPU): the library loads, exports every
symbol include/ring_attn.h declares, sizes workspaces, and rejects invalid
arguments before touching a device."""
import ctypes
import os
import re

import pytest

import blockwise_ring_attention_attn_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return ra.load()


def test_exports_every_header_symbol(lib):
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert sorted(ra.EXPORTS) == names


def test_version(lib):
    assert b"gfx950" in lib.ra_version()


def test_ws_bytes():
    # C2: two staging buffers of K+V (bf16) plus fp32 m, l, o
    B, H, N, d, P = 1, 32, 32768, 128, 8
    kv = B * H * N * d * 2
    state = B * H * N * 4 * 2 + B * H * N * d * 4
    assert ra.ring_attn_fwd_ws_bytes(B, H, H, N, d, P, ra.RA_BF16) == 4 * kv + state
    assert ra.ring_attn_fwd_ws_bytes(B, H, H, N, d, 1, ra.RA_BF16) == 0
    assert ra.load().ring_attn_fwd_ws_bytes(B, H, H, N + 1, d, P, ra.RA_BF16) == 0
    assert ra.load().ring_attn_decode_ws_bytes(16, 32, 8, 262144, 128, 8) > 0


def _fwd(lib, **kw):
    a = dict(q=1, k=1, v=1, out=1, lse=1, B=1, H=2, Hkv=1, N=64, d=64, P=4, causal=1, layout=0,
             scale=0.125, dtype=1, stream=None, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    return lib.ring_attn_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"],
                             a["d"], a["P"], a["causal"], a["layout"], a["scale"], a["dtype"], a["stream"],
                             a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("kw,frag", [
    (dict(q=None), "null"),
    (dict(N=65), "multiple of P"),
    (dict(H=3, Hkv=2), "multiple of Hkv"),
    (dict(d=96), "64 or 128"),
    (dict(P=0), "P must be"),
    (dict(P=65, N=65 * 4), "P must be"),
    (dict(ws_bytes=16), "workspace too small"),
    (dict(ws=None), "null workspace"),
    (dict(ws=255), "aligned"),
    (dict(layout=7), "layout"),
    (dict(layout=2, N=68), "multiple of 2P"),
    (dict(dtype=9), "dtype"),
    (dict(scale=0.0), "scale"),
    (dict(scale=float("nan")), "scale"),
])
def test_fwd_rejects_invalid(lib, kw, frag):
    assert _fwd(lib, **kw) == ra.RA_EINVAL
    assert frag in lib.ra_last_error().decode()


def test_step_rejects_invalid(lib):
    md = ra.ra_mask_desc(1, 2, 1, 64, 16, 16, 0.125, ra.RA_BF16, 1, 0, 4, 5, 0)  # q_rank >= P
    st = lib.ring_attn_step(1, ra.ra_kv_block(1, 1), 1, 1, 1, ctypes.byref(md), None)
    assert st == ra.RA_EINVAL and b"ring" in lib.ra_last_error()
    assert lib.ring_attn_step(1, ra.ra_kv_block(1, 1), 1, 1, 1, None, None) == ra.RA_EINVAL
    md = ra.ra_mask_desc(1, 2, 1, 64, 16, 8, 0.125, ra.RA_BF16, 1, 1, 4, 1, 0)  # striped causal Lq != Lkv
    assert lib.ring_attn_step(1, ra.ra_kv_block(1, 1), 1, 1, 1, ctypes.byref(md), None) == ra.RA_EINVAL
    md = ra.ra_mask_desc(1, 2, 1, 64, 15, 15, 0.125, ra.RA_BF16, 1, 2, 4, 1, 0)  # zigzag causal, odd length
    assert lib.ring_attn_step(1, ra.ra_kv_block(1, 1), 1, 1, 1, ctypes.byref(md), None) == ra.RA_EINVAL
    assert b"zigzag" in lib.ra_last_error()


def test_merge_decode_reject_invalid(lib):
    assert lib.lse_merge(None, 1, 1, 1, 4, 8, None) == ra.RA_EINVAL
    assert lib.lse_merge(1, 1, 1, 1, 4, 0, None) == ra.RA_EINVAL
    assert lib.ring_attn_finalize(1, 1, 1, 1, 1, 4, 2000, 1, None) == ra.RA_EINVAL
    # decode: f32 unsupported, group > 16, L % P
    assert lib.ring_attn_decode(1, 1, 1, 1, 1, 1, 32, 1, 64, 64, 4, 0.1, 0, None, 256, 1 << 30) == ra.RA_EUNSUPPORTED
    assert lib.ring_attn_decode(1, 1, 1, 1, 1, 1, 32, 1, 64, 64, 4, 0.1, 1, None, 256, 1 << 30) == ra.RA_EINVAL
    assert lib.ring_attn_decode(1, 1, 1, 1, 1, 1, 4, 1, 66, 64, 4, 0.1, 1, None, 256, 1 << 30) == ra.RA_EINVAL


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        ra.load(str(tmp_path / "missing.so"))


def _share(lib, **kw):
    a = dict(q=1, k=1, v=1, out=1, lse=1, B=1, H=2, Hkv=1, N=64, d=64, P=4, rank=3, causal=1, layout=0,
             scale=0.125, dtype=1, stream=None, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    return lib.ring_attn_fwd_share(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"],
                                   a["d"], a["P"], a["rank"], a["causal"], a["layout"], a["scale"], a["dtype"],
                                   a["stream"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("kw,frag", [
    (dict(lse=None), "null"),
    (dict(rank=4), "rank"),
    (dict(rank=-1), "rank"),
    (dict(N=66), "multiple of P"),
    (dict(d=80), "64 or 128"),
    (dict(ws_bytes=16), "workspace too small"),
    (dict(ws=8), "aligned"),
    (dict(layout=2, N=68), "multiple of 2P"),
])
def test_share_rejects_invalid(lib, kw, frag):
    assert _share(lib, **kw) == ra.RA_EINVAL
    assert frag in lib.ra_last_error().decode()


def _bwd(lib, **kw):
    a = dict(q=1, k=1, v=1, out=1, dout=1, lse=1, dq=1, dk=1, dv=1, B=1, H=2, Hkv=1, N=64, d=64, P=4, causal=1,
             layout=0, scale=0.125, dtype=1, stream=None, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    return lib.ring_attn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                             a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["P"], a["causal"], a["layout"], a["scale"],
                             a["dtype"], a["stream"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("kw,status,frag", [
    (dict(dout=None), ra.RA_EINVAL, "null"),
    (dict(dv=None), ra.RA_EINVAL, "null"),
    (dict(N=65), ra.RA_EINVAL, "multiple of P"),
    (dict(H=3, Hkv=2), ra.RA_EINVAL, "multiple of Hkv"),
    (dict(P=65, N=65 * 4), ra.RA_EINVAL, "P must be"),
    (dict(dtype=0), ra.RA_EUNSUPPORTED, "bf16 only"),
    (dict(ws_bytes=16), ra.RA_EINVAL, "workspace too small"),
    (dict(ws=None), ra.RA_EINVAL, "null workspace"),
    (dict(ws=100), ra.RA_EINVAL, "aligned"),
])
def test_bwd_rejects_invalid(lib, kw, status, frag):
    assert _bwd(lib, **kw) == status
    assert frag in lib.ra_last_error().decode()


def test_bwd_ws_bytes_cover_fp32_gradients():
    # fp32 accumulators for dq (B H N d), dk and dv (B Hkv N d), plus lse2 and delta (B H N)
    B, H, Hkv, N, d, P = 1, 32, 8, 32768, 128, 8
    need = 4 * (B * H * N * d + 2 * B * Hkv * N * d + 2 * B * H * N)
    got = ra.load().ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16)
    assert need <= got <= need + (1 << 16)


@pytest.mark.parametrize("kw,frag", [
    (dict(q=8), "16-byte aligned"),
    (dict(out=256 + 4), "16-byte aligned"),
    (dict(lse=258), "4-byte aligned"),
])
def test_fwd_rejects_misaligned_tensors(lib, kw, frag):
    base = dict(q=256, k=512, v=768, out=1024, lse=1280)
    base.update(kw)
    assert _fwd(lib, **base) == ra.RA_EINVAL
    assert frag in lib.ra_last_error().decode()


def test_other_entry_points_reject_misaligned_tensors(lib):
    t = dict(q=256, k=512, v=768, out=1024, lse=1280)
    assert _share(lib, **dict(t, v=776)) == ra.RA_EINVAL
    assert b"16-byte" in lib.ra_last_error()
    assert _bwd(lib, **dict(t, dout=2048, dq=2304, dk=2568, dv=2816)) == ra.RA_EINVAL
    assert b"16-byte" in lib.ra_last_error()
    md = ra.ra_mask_desc(1, 2, 1, 64, 16, 16, 0.125, ra.RA_BF16, 1, 0, 4, 1, 0)
    assert lib.ring_attn_step(256, ra.ra_kv_block(512, 768), 1024, 1280, 1544, ctypes.byref(md), None) == ra.RA_EINVAL
    assert b"16-byte" in lib.ra_last_error()
    assert lib.ring_attn_step(256, ra.ra_kv_block(512, 768), 1026, 1280, 1536, ctypes.byref(md), None) == ra.RA_EINVAL
    assert b"4-byte" in lib.ra_last_error()
    assert lib.ring_attn_decode(264, 512, 768, 1024, 1280, 1, 4, 1, 64, 64, 4, 0.1, 1, None, 256, 1 << 30) == ra.RA_EINVAL
    assert b"16-byte" in lib.ra_last_error()


def test_merge_and_finalize_of_zero_rows_are_no_ops(lib):
    assert lib.lse_merge(None, None, None, None, 0, 8, None) == ra.RA_OK
    assert lib.ring_attn_finalize(None, None, None, None, None, 0, 128, 1, None) == ra.RA_OK
    assert lib.lse_merge(None, None, None, None, -1, 8, None) == ra.RA_EINVAL
    assert lib.ring_attn_finalize(None, None, None, None, None, 0, 128, 9, None) == ra.RA_EINVAL
