"""ring_attn_decode_noalloc (static scratch, no workspace) against
ring_attn_decode (caller workspace): the same kernels, so the results must
be bit-identical, and both within the tolerance of the fp64 oracle (bf16
and fp32).
Two calls in a row, the second with a smaller input (the scratch keeps the
first call's partials; every call rewrites the ones it reads)."""
import pytest

import blockwise_ring_attention_attn_amd as ra
import oracle
import synth
from _util import assert_close, from_dev, host_vals, to_dev

pytestmark = pytest.mark.gpu


def _one(seed, B, H, Hkv, L, d, P, dtype="bf16"):
    import torch
    print(f"\n[noalloc] B={B} H={H}/{Hkv} L={L} d={d} P={P} {dtype}", flush=True)
    q, k, v = synth.qkv(seed, B, H, Hkv, L, d, dtype, Nq=1)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out_ws, lse_ws = ra.ring_attn_decode(qd, kd, vd, P=P)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H), float("nan"), device=qd.device)
    ra.ring_attn_decode_noalloc(qd, kd, vd, P=P, out=out, lse=lse)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(out.view(bits), out_ws.view(bits))
    assert torch.equal(lse, lse_ws)
    Ow, Lw = oracle.decode(host_vals(q, dtype), host_vals(k, dtype), host_vals(v, dtype))
    assert_close(from_dev(out), from_dev(lse), Ow, Lw[:, :, 0], dtype, f"decode_noalloc B={B} L={L} {dtype}")


def test_noalloc_matches_workspace_decode_twice():
    # 16 x 32 heads, P = 8: 128 partials per head (34 MB of scratch, as for a
    # 262144-key cache), then a smaller problem that reuses the array
    _one(31, 16, 32, 8, 8192, 128, 8)
    _one(32, 2, 8, 2, 8 * 1000, 64, 8)


def test_noalloc_fp32_matches_workspace_decode_twice():
    _one(33, 4, 8, 2, 4 * 2048, 128, 4, "f32")
    _one(34, 1, 4, 4, 8 * 100, 64, 8, "f32")
