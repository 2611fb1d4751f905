"""ring_attn_decode_noalloc (static scratch, no workspace) against
ring_attn_decode (caller workspace): the same kernels, so the results must
be bit-identical, and both within the bf16 tolerance of the fp64 oracle.
Two calls in a row, the second with a smaller input (the scratch keeps the
first call's partials; every call rewrites the ones it reads)."""
import numpy as np
import pytest

import blockwise_ring_attention_attn_amd as ra
import oracle
import synth
from _util import assert_close, from_dev, host_vals, to_dev

pytestmark = pytest.mark.gpu


def _one(seed, B, H, Hkv, L, d, P):
    import torch
    print(f"\n[noalloc] B={B} H={H}/{Hkv} L={L} d={d} P={P}", flush=True)
    q, k, v = synth.qkv(seed, B, H, Hkv, L, d, "bf16", Nq=1)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    out_ws, lse_ws = ra.ring_attn_decode(qd, kd, vd, P=P)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H), float("nan"), device=qd.device)
    ra.ring_attn_decode_noalloc(qd, kd, vd, P=P, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_ws.view(torch.int16))
    assert torch.equal(lse, lse_ws)
    Ow, Lw = oracle.decode(host_vals(q, "bf16"), host_vals(k, "bf16"), host_vals(v, "bf16"))
    assert_close(from_dev(out), from_dev(lse), Ow, Lw[:, :, 0], "bf16", f"decode_noalloc B={B} L={L}")


def test_noalloc_matches_workspace_decode_twice():
    # 16 x 32 heads, P = 8: 128 partials per head (34 MB of scratch, as for a
    # 262144-key cache), then a smaller problem that reuses the array
    _one(31, 16, 32, 8, 8192, 128, 8)
    _one(32, 2, 8, 2, 8 * 1000, 64, 8)
