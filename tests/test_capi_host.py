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


SIZE_MAX = (1 << 64) - 1


def test_ws_bytes():
    # C2: two staging buffers of K+V (bf16) plus fp32 m, l, o
    B, H, N, d, P = 1, 32, 32768, 128, 8
    kv = B * H * N * d * 2
    state = B * H * N * 4 * 2 + B * H * N * d * 4
    assert ra.ring_attn_fwd_ws_bytes(B, H, H, N, d, P, ra.RA_BF16) == 4 * kv + state
    assert ra.ring_attn_fwd_ws_bytes(B, H, H, N, d, 1, ra.RA_BF16) == 0  # valid, nothing to stage
    assert ra.load().ring_attn_decode_ws_bytes(16, 32, 8, 262144, 128, 8) > 0


@pytest.mark.parametrize("args,frag", [
    ((1, 32, 32, 32768 + 1, 128, 8, 1), "multiple of P"),
    ((1, 32, 32, 32768, 96, 8, 1), "64 or 128"),
    ((1, 3, 2, 32768, 128, 8, 1), "multiple of Hkv"),
    ((1, 32, 32, 32768, 128, 8, 7), "dtype"),
    ((0, 32, 32, 32768, 128, 8, 1), ">= 1"),
    ((1, 32, 32, 32768, 128, 0, 1), "P must be"),
    ((1, 1, 1, 8 << 24, 128, 8, 1), "below 2 GiB"),  # one 2^24-row bf16 block is 4 GiB
])
def test_ws_queries_flag_invalid_arguments(lib, args, frag):
    """Invalid arguments give SIZE_MAX (not 0, which means 'no workspace
    needed') with the launch's own message."""
    assert lib.ring_attn_fwd_ws_bytes(*args) == SIZE_MAX
    assert frag in lib.ra_last_error().decode()
    assert lib.ring_attn_fwd_share_ws_bytes(*args) == SIZE_MAX
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_fwd_ws_bytes(*args)


def test_other_ws_queries_flag_invalid_arguments(lib):
    assert lib.ring_attn_bwd_ws_bytes(1, 2, 1, 64, 64, 4, 7) == SIZE_MAX
    assert b"unknown dtype" in lib.ra_last_error()
    assert lib.ring_attn_bwd_ws_bytes(1, 2, 1, 65, 64, 4, ra.RA_BF16) == SIZE_MAX
    assert lib.ring_attn_bwd_ws_bytes(1, 1, 1, 1 << 24, 128, 8, ra.RA_BF16) == SIZE_MAX  # 4 GiB plane
    assert b"below 2 GiB" in lib.ra_last_error()
    assert lib.ring_attn_decode_ws_bytes(1, 32, 1, 64, 96, 4) == SIZE_MAX  # d = 96
    assert lib.ring_attn_decode_ws_bytes(1, 4, 1, 66, 64, 4) == SIZE_MAX
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_decode_ws_bytes(1, 4, 1, 66, 64, 4)


def test_ws_queries_report_sizes_beyond_the_address_space(lib):
    """B*H*N*d*4 bytes past 2^48 (the device's virtual address width) or past
    2^64: SIZE_MAX from the query, RA_ENOMEM from the launch."""
    B, H, N, d, P = 1 << 20, 1 << 10, 1 << 28, 128, 64
    assert lib.ring_attn_fwd_ws_bytes(B, H, H, N, d, P, ra.RA_BF16) == SIZE_MAX
    assert b"address space" in lib.ra_last_error()
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_fwd_ws_bytes(B, H, H, N, d, P, ra.RA_BF16)
    assert e.value.status == ra.RA_ENOMEM
    st = lib.ring_attn_fwd(256, 256, 256, 256, 256, B, H, H, N, d, P, 1, 0, 0.1, ra.RA_BF16, None, 256, 1 << 40)
    assert st == ra.RA_ENOMEM and b"address space" in lib.ra_last_error()
    st = lib.ring_attn_bwd(256, 256, 256, 256, 256, 256, 256, 256, 256, 1 << 20, 1 << 12, 1 << 12, 1 << 22, 128, 8,
                           1, 0, 0.1, ra.RA_BF16, None, 256, 1 << 40)
    assert st == ra.RA_ENOMEM
    assert lib.ring_attn_decode_ws_bytes(1 << 20, 1 << 16, 1 << 12, 64 * 128, 128, 64) == SIZE_MAX
    assert b"address space" in lib.ra_last_error()


def test_large_planes_are_accepted_where_the_kernels_allow():
    """A 9,437,184-token kv plane (2.4 GB per head in bf16) passes the
    argument checks of the forward (contiguous, striped: its first step is
    staged), the share and decode; they stop at the workspace check here."""
    lib = ra.load()
    N, d, P = 9437184, 128, 8
    for layout in (0, 1, 2):
        st = lib.ring_attn_fwd(256, 256, 256, 256, 256, 1, 1, 1, N, d, P, 1, layout, 0.1, ra.RA_BF16, None, 256, 16)
        assert st == ra.RA_EINVAL and b"workspace too small" in lib.ra_last_error(), layout
        st = lib.ring_attn_fwd_share(256, 256, 256, 256, 256, 1, 1, 1, N, d, P, 7, 1, layout, 0.1, ra.RA_BF16,
                                     None, 256, 16)
        assert st == ra.RA_EINVAL and b"workspace too small" in lib.ra_last_error(), layout
    st = lib.ring_attn_decode(256, 256, 256, 256, 256, 1, 4, 1, N, d, P, 0.1, ra.RA_BF16, None, 256, 16)
    assert st == ra.RA_EINVAL and b"workspace too small" in lib.ra_last_error()
    assert 0 < lib.ring_attn_decode_ws_bytes(1, 4, 1, N, d, P) < SIZE_MAX
    assert 0 < lib.ring_attn_fwd_share_ws_bytes(1, 1, 1, N, d, P, ra.RA_BF16) < SIZE_MAX


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


def test_bwd_step_and_prep_reject_invalid(lib):
    kvb = ra.ra_kv_block(256, 512)
    md = ra.ra_mask_desc(1, 2, 1, 64, 16, 16, 0.125, ra.RA_BF16, 1, 0, 4, 1, 0)
    ok = dict(q=768, do=1024, rs=1280, dq=1536, dk=1792, dv=2048)

    def step(md_ref, **kw):
        a = dict(ok, **kw)
        return lib.ring_attn_bwd_step(a["q"], a["do"], a["rs"], kvb, a["dq"], a["dk"], a["dv"], md_ref, None)

    assert step(None) == ra.RA_EINVAL and b"mask_desc" in lib.ra_last_error()
    assert step(ctypes.byref(md), rs=None) == ra.RA_EINVAL and b"null" in lib.ra_last_error()
    assert step(ctypes.byref(md), dv=None) == ra.RA_EINVAL
    assert step(ctypes.byref(md), dk=1800) == ra.RA_EINVAL and b"16-byte" in lib.ra_last_error()
    bad = ra.ra_mask_desc(1, 2, 1, 64, 16, 16, 0.125, ra.RA_BF16, 1, 0, 4, 5, 0)       # q_rank >= P
    assert step(ctypes.byref(bad)) == ra.RA_EINVAL and b"ring" in lib.ra_last_error()
    bad = ra.ra_mask_desc(1, 2, 1, 96, 16, 16, 0.125, ra.RA_BF16, 1, 0, 4, 1, 0)       # d
    assert step(ctypes.byref(bad)) == ra.RA_EINVAL and b"64 or 128" in lib.ra_last_error()
    bad = ra.ra_mask_desc(1, 2, 1, 64, 15, 15, 0.125, ra.RA_BF16, 1, 2, 4, 1, 0)       # zigzag causal, odd length
    assert step(ctypes.byref(bad)) == ra.RA_EINVAL and b"zigzag" in lib.ra_last_error()
    bad = ra.ra_mask_desc(1, 1, 1, 128, 1 << 23, 16, 0.125, ra.RA_BF16, 0, 0, 1, 0, 0)  # 2 GiB query plane
    assert step(ctypes.byref(bad)) == ra.RA_EINVAL and b"query block plane" in lib.ra_last_error()
    # prep: rows, d, dtype, pointers, alignment; zero rows is a no-op
    assert lib.ring_attn_bwd_prep(256, 512, 768, 1024, -1, 64, 1, None) == ra.RA_EINVAL
    assert lib.ring_attn_bwd_prep(256, 512, 768, 1024, 8, 80, 1, None) == ra.RA_EINVAL
    assert lib.ring_attn_bwd_prep(256, 512, 768, 1024, 8, 64, 5, None) == ra.RA_EINVAL
    assert lib.ring_attn_bwd_prep(256, None, 768, 1024, 8, 64, 1, None) == ra.RA_EINVAL
    assert lib.ring_attn_bwd_prep(256, 512, 768, 1032, 8, 64, 1, None) == ra.RA_EINVAL
    assert b"16-byte" in lib.ra_last_error()
    assert lib.ring_attn_bwd_prep(None, None, None, None, 0, 64, 1, None) == ra.RA_OK


def test_binding_rejects_bad_backward_step_arguments():
    import torch
    f32 = torch.float32
    q, k = _t(1, 2, 16, 64), _t(1, 1, 16, 64)
    rs = _t(1, 2, 16, 2, dtype=f32)
    dq, dk = _t(1, 2, 16, 64, dtype=f32), _t(1, 1, 16, 64, dtype=f32)
    with pytest.raises(ValueError, match="rowstat must have shape"):
        ra.ring_attn_bwd_step(q, k, k, q, _t(1, 2, 16, dtype=f32), dq, dk, dk.clone(), causal=True)
    with pytest.raises(TypeError, match="dq_acc must be"):
        ra.ring_attn_bwd_step(q, k, k, q, rs, q, dk, dk.clone(), causal=True)
    with pytest.raises(ValueError, match="dk_acc must have shape"):
        ra.ring_attn_bwd_step(q, k, k, q, rs, dq, _t(1, 2, 16, 64, dtype=f32), dk, causal=True)
    with pytest.raises(ValueError, match="dout_blk must have shape"):
        ra.ring_attn_bwd_step(q, k, k, _t(1, 2, 8, 64), rs, dq, dk, dk.clone(), causal=True)
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_bwd_step(q, k, k, q, rs, dq, dk, dk.clone(), causal=True)
    with pytest.raises(ValueError, match="lse must have shape"):
        ra.ring_attn_bwd_prep(q, q, _t(1, 2, 8, dtype=f32))
    with pytest.raises(TypeError, match="dout must be"):
        ra.ring_attn_bwd_prep(q, q.float(), _t(1, 2, 16, dtype=f32))
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_bwd_prep(q, q, _t(1, 2, 16, dtype=f32))


def test_merge_decode_reject_invalid(lib):
    assert lib.lse_merge(None, 1, 1, 1, 4, 8, None) == ra.RA_EINVAL
    assert lib.lse_merge(1, 1, 1, 1, 4, 0, None) == ra.RA_EINVAL
    assert lib.ring_attn_finalize(1, 1, 1, 1, 1, 4, 2000, 1, None) == ra.RA_EINVAL
    # decode: unknown dtype, H % Hkv, d (bf16 and fp32), L % P
    assert lib.ring_attn_decode(1, 1, 1, 1, 1, 1, 4, 1, 64, 64, 4, 0.1, 7, None, 256, 1 << 30) == ra.RA_EINVAL
    assert b"unknown dtype" in lib.ra_last_error()
    assert lib.ring_attn_decode(1, 1, 1, 1, 1, 1, 32, 3, 64, 64, 4, 0.1, 1, None, 256, 1 << 30) == ra.RA_EINVAL
    assert lib.ring_attn_decode(1, 1, 1, 1, 1, 1, 32, 1, 64, 96, 4, 0.1, 0, None, 256, 1 << 30) == ra.RA_EINVAL
    assert lib.ring_attn_decode(1, 1, 1, 1, 1, 1, 32, 1, 64, 96, 4, 0.1, 1, None, 256, 1 << 30) == ra.RA_EINVAL
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
    (dict(dtype=7), ra.RA_EINVAL, "unknown dtype"),
    (dict(ws_bytes=16), ra.RA_EINVAL, "workspace too small"),
    (dict(ws=None), ra.RA_EINVAL, "null workspace"),
    (dict(ws=100), ra.RA_EINVAL, "aligned"),
])
def test_bwd_rejects_invalid(lib, kw, status, frag):
    assert _bwd(lib, **kw) == status
    assert frag in lib.ra_last_error().decode()


def test_bwd_ws_bytes_cover_fp32_gradients():
    # fp32 accumulators for dq (B H N d), dk and dv (B Hkv N d), plus lse2 and delta (B H N);
    # for P > 1 two bf16 staging buffers of K and V (the reverse ring's exchange)
    B, H, Hkv, N, d, P = 1, 32, 8, 32768, 128, 8
    need = 4 * (B * H * N * d + 2 * B * Hkv * N * d + 2 * B * H * N)
    stage = 2 * 2 * (B * Hkv * N * d * 2)
    got = ra.load().ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16)
    assert need + stage <= got <= need + stage + (1 << 16)
    got1 = ra.load().ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, 1, ra.RA_BF16)
    assert need <= got1 <= need + (1 << 16)


def _bwd_share(lib, **kw):
    a = dict(q=1, k=1, v=1, out=1, dout=1, lse=1, dq=1, dk=1, dv=1, B=1, H=2, Hkv=1, N=64, d=64, P=4, rank=1,
             causal=1, layout=0, scale=0.125, dtype=1, stream=None, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    return lib.ring_attn_bwd_share(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"],
                                   a["dv"], a["B"], a["H"], a["Hkv"], a["N"], a["d"], a["P"], a["rank"],
                                   a["causal"], a["layout"], a["scale"], a["dtype"], a["stream"], a["ws"],
                                   a["ws_bytes"])


@pytest.mark.parametrize("kw,frag", [
    (dict(lse=None), "null"),
    (dict(dk=None), "null"),
    (dict(rank=4), "rank 4 out of"),
    (dict(rank=-1), "rank -1 out of"),
    (dict(N=66), "multiple of P"),
    (dict(d=96), "64 or 128"),
    (dict(layout=2, N=68), "multiple of 2P"),
    (dict(ws_bytes=16), "workspace too small"),
    (dict(ws=None), "null workspace"),
    (dict(ws=100), "aligned"),
    (dict(q=256, k=512, v=776, out=1024, dout=1280, dq=1536, dk=1792, dv=2048, lse=2304), "16-byte"),
])
def test_bwd_share_rejects_invalid(lib, kw, frag):
    assert _bwd_share(lib, **kw) == ra.RA_EINVAL
    assert frag in lib.ra_last_error().decode()


def test_bwd_share_ws_bytes():
    """One device's share of the backward holds two staging slots of one kv
    block (K and V), the fp32 dq accumulator and the row statistics of the
    rank's N/P rows; nothing for dk / dv (each step writes its block's
    gradients directly)."""
    lib = ra.load()
    for dtype, es in ((ra.RA_BF16, 2), (ra.RA_F32, 4)):
        B, H, Hkv, N, d, P = 1, 4, 1, 8 * 131072, 128, 8
        Bl = N // P
        need = 4 * (B * H * Bl * d + 2 * B * H * Bl) + 2 * 2 * (B * Hkv * Bl * d * es)
        got = lib.ring_attn_bwd_share_ws_bytes(B, H, Hkv, N, d, P, dtype)
        assert need <= got <= need + (1 << 16)
        got1 = lib.ring_attn_bwd_share_ws_bytes(B, H, Hkv, N // P, d, 1, dtype)
        assert 4 * (B * H * Bl * d + 2 * B * H * Bl) <= got1 <= 4 * (B * H * Bl * d + 2 * B * H * Bl) + (1 << 16)
    assert lib.ring_attn_bwd_share_ws_bytes(1, 1, 1, 1 << 24, 128, 8, ra.RA_BF16) == SIZE_MAX   # 4 GiB kv plane


def test_binding_rejects_bad_backward_share_arguments():
    import torch
    f32 = torch.float32
    qs, k = _t(1, 2, 16, 64), _t(1, 1, 64, 64)          # rank block of N / P = 16 rows, P = 4
    lse = _t(1, 2, 16, dtype=f32)
    with pytest.raises(ValueError, match="q must hold N / P rows"):
        ra.ring_attn_bwd_share(_t(1, 2, 32, 64), k, k, _t(1, 2, 32, 64), _t(1, 2, 32, 64), _t(1, 2, 32, dtype=f32),
                               P=4, rank=1, causal=True)
    with pytest.raises(ValueError, match="out must have shape"):
        ra.ring_attn_bwd_share(qs, k, k, _t(1, 2, 64, 64), qs, lse, P=4, rank=1, causal=True)
    with pytest.raises(ValueError, match="lse must have shape"):
        ra.ring_attn_bwd_share(qs, k, k, qs, qs, _t(1, 2, 64, dtype=f32), P=4, rank=1, causal=True)
    with pytest.raises(ValueError, match="dk must have shape"):
        ra.ring_attn_bwd_share(qs, k, k, qs, qs, lse, P=4, rank=1, causal=True, dk=_t(1, 1, 16, 64))
    with pytest.raises(TypeError, match="dv must be"):
        ra.ring_attn_bwd_share(qs, k, k, qs, qs, lse, P=4, rank=1, causal=True, dv=_t(1, 1, 64, 64, dtype=f32))
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_bwd_share(qs, k, k, qs, qs, lse, P=4, rank=1, causal=True)


def test_decode_ws_bytes_count_query_head_sub_groups():
    """Query heads beyond 16 per kv head are decoded in sub-groups of 16; the
    partials stay one per (batch, head, split), so the workspace for a
    multi-query group of 32 equals that of 32 kv heads with one query each
    at the same number of splits per ring block."""
    lib = ra.load()
    nb_mqa = lib.ring_attn_decode_ws_bytes(2, 32, 1, 4096, 128, 4)
    assert nb_mqa not in (0, SIZE_MAX)
    nb_mha = lib.ring_attn_decode_ws_bytes(2, 32, 32, 4096, 128, 4)
    assert nb_mqa <= nb_mha   # fewer workgroup planes -> at least as many splits per block, never more partials


def test_bwd_fp32_ws_bytes_and_plane_limit():
    """The fp32 backward stages K and V in fp32 (4-byte elements) and, since
    its kernels address with 64-bit pointers, has no 2 GiB plane limit."""
    B, H, Hkv, N, d, P = 1, 4, 2, 4096, 64, 4
    need = 4 * (B * H * N * d + 2 * B * Hkv * N * d + 2 * B * H * N)
    stage = 2 * 2 * (B * Hkv * N * d * 4)
    got = ra.load().ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_F32)
    assert need + stage <= got <= need + stage + (1 << 16)
    lib = ra.load()
    assert lib.ring_attn_bwd_ws_bytes(1, 1, 1, 1 << 24, 128, 8, ra.RA_F32) not in (0, SIZE_MAX)  # 8 GiB plane


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


# ---------------------------------------------------------------------------
# The Python binding checks every tensor before a pointer reaches the
# library: dtype, exact shape and contiguity first, then the device.
# (Host tensors here: each case must fail on the property it breaks.)
# ---------------------------------------------------------------------------
def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_rejects_bad_forward_arguments():
    import torch
    q, k, v = _t(1, 4, 64, 64), _t(1, 2, 64, 64), _t(1, 2, 64, 64)
    with pytest.raises(TypeError, match="k must be"):
        ra.ring_attn_fwd(q, k.float(), v, P=4, causal=True)
    with pytest.raises(ValueError, match="v must have shape"):
        ra.ring_attn_fwd(q, k, _t(1, 2, 64, 128), P=4, causal=True)
    with pytest.raises(ValueError, match="out must have shape"):
        ra.ring_attn_fwd(q, k, v, P=4, causal=True, out=_t(1, 4, 32, 64))
    with pytest.raises(TypeError, match="out must be"):
        ra.ring_attn_fwd(q, k, v, P=4, causal=True, out=_t(1, 4, 64, 64, dtype=torch.float32))
    with pytest.raises(TypeError, match="lse must be"):
        ra.ring_attn_fwd(q, k, v, P=4, causal=True, lse=_t(1, 4, 64))
    with pytest.raises(ValueError, match="lse must have shape"):
        ra.ring_attn_fwd(q, k, v, P=4, causal=True, lse=_t(1, 4, 65, dtype=torch.float32))
    with pytest.raises(ValueError, match="contiguous"):
        ra.ring_attn_fwd(q, k, v, P=4, causal=True, out=_t(1, 4, 64, 64).transpose(2, 3))
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_fwd(q, k, v, P=4, causal=True)
    with pytest.raises(ValueError, match="q must hold N / P rows"):
        ra.ring_attn_fwd_share(_t(1, 4, 32, 64), k, v, P=4, rank=3, causal=True)


def test_binding_rejects_bad_step_merge_finalize_decode_backward_arguments():
    import torch
    f32 = torch.float32
    q, k, v = _t(1, 2, 16, 64), _t(1, 1, 16, 64), _t(1, 1, 16, 64)
    m, l, o = _t(1, 2, 16, dtype=f32), _t(1, 2, 16, dtype=f32), _t(1, 2, 16, 64, dtype=f32)
    with pytest.raises(TypeError, match="o must be"):
        ra.ring_attn_step(q, k, v, m, l, o.bfloat16(), causal=True)
    with pytest.raises(ValueError, match="m must have shape"):
        ra.ring_attn_step(q, k, v, _t(1, 2, 15, dtype=f32), l, o, causal=True)
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_step(q, k, v, m, l, o, causal=True)
    with pytest.raises(TypeError, match="o_a must be"):
        ra.lse_merge(o.bfloat16(), m, o, l)
    with pytest.raises(ValueError, match="lse_b must have shape"):
        ra.lse_merge(o, m, o.clone(), _t(1, 2, 17, dtype=f32))
    with pytest.raises(ValueError, match="device tensor"):
        ra.lse_merge(o, m, o.clone(), l)
    with pytest.raises(ValueError, match="l must have shape"):
        ra.ring_attn_finalize(m, _t(2, 16, dtype=f32), o)
    with pytest.raises(ValueError, match="out must have shape"):
        ra.ring_attn_finalize(m, l, o, out=_t(1, 2, 16, 32))
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_finalize(m, l, o)
    qd, kd, vd = _t(2, 8, 1, 128), _t(2, 2, 256, 128), _t(2, 2, 256, 128)
    with pytest.raises(ValueError, match=r"\[B, H, 1, d\]"):
        ra.ring_attn_decode(_t(2, 8, 2, 128), kd, vd, P=2)
    with pytest.raises(TypeError, match="v must be"):
        ra.ring_attn_decode(qd, kd, vd.float(), P=2)
    with pytest.raises(ValueError, match="lse must have shape"):
        ra.ring_attn_decode(qd, kd, vd, P=2, lse=_t(2, 8, 1, dtype=f32))
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_decode(qd, kd, vd, P=2)
    qb, kb = _t(1, 2, 64, 64), _t(1, 1, 64, 64)
    lse = _t(1, 2, 64, dtype=f32)
    with pytest.raises(ValueError, match="dk must have shape"):
        ra.ring_attn_bwd(qb, kb, kb, qb, qb, lse, P=4, causal=True, dk=_t(1, 2, 64, 64))
    with pytest.raises(TypeError, match="lse must be"):
        ra.ring_attn_bwd(qb, kb, kb, qb, qb, lse.bfloat16(), P=4, causal=True)
    with pytest.raises(TypeError, match="k must be"):
        ra.ring_attn_bwd(qb.float(), kb, kb, qb.float(), qb.float(), lse, P=4, causal=True)
    with pytest.raises(TypeError, match="dq must be"):
        ra.ring_attn_bwd(qb.float(), kb.float(), kb.float(), qb.float(), qb.float(), lse, P=4, causal=True, dq=qb)
    with pytest.raises(ValueError, match="device tensor"):
        ra.ring_attn_bwd(qb, kb, kb, qb, qb, lse, P=4, causal=True)


def test_decode_noalloc_rejects_what_the_static_scratch_cannot_hold(lib):
    """ring_attn_decode_noalloc keeps its partials in a 64 MiB static array:
    a problem whose partials need more is refused before any device call
    (64 sequences x 16 heads x 1024 partials x 129 floats)."""
    need = ra.ring_attn_decode_ws_bytes(64, 16, 16, 64 * 4096, 128, 64)
    assert need > 64 << 20
    st = lib.ring_attn_decode_noalloc(256, 256, 256, 256, 256, 64, 16, 16, 64 * 4096, 128, 64, 0.1, ra.RA_BF16, None)
    assert st == ra.RA_EINVAL and b"static scratch" in lib.ra_last_error()
    # and the decode workload of 16 sequences x 262144 keys fits (34 MB)
    assert ra.ring_attn_decode_ws_bytes(16, 32, 8, 262144, 128, 8) <= 64 << 20
    assert lib.ring_attn_decode_noalloc(None, 1, 1, 1, 1, 16, 32, 8, 262144, 128, 8, 0.1, ra.RA_BF16, None) == ra.RA_EINVAL
