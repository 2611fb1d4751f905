"""GPU tests of the ring driver's stream ordering, workspace hygiene and
resumable state (the step state between ring steps is a checkpoint).

Stream ordering: the staging copy for step s + 1 must wait for step s - 1's
kernel (it overwrites what that step read) and step s's kernel must wait for
its copy.  A bounded spin injected before every step kernel lets copies run
ahead; one injected before every copy makes the kernels wait.  Either way the
result must be bitwise the one without delays.
"""
import numpy as np
import pytest

import blockwise_ring_attention_attn_amd as ra
import synth
from _util import from_dev, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, Hkv, N, d):
    print(f"\n[driver] seed={seed} B={B} H={H}/{Hkv} N={N} d={d}", flush=True)
    q, k, v = synth.qkv(seed, B, H, Hkv, N, d, "bf16")
    return to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("delays", [(2000, 0), (0, 2000)])
def test_fwd_stream_order_under_delays(layout, delays):
    qd, kd, vd = _inputs(21, 1, 4, 2, 8 * 256, 128)
    ref = ra.ring_attn_fwd(qd, kd, vd, P=8, causal=True, layout=layout)
    ref = (from_dev(ref[0]), from_dev(ref[1]))
    try:
        ra.debug_set_delays(*delays)
        got = ra.ring_attn_fwd(qd, kd, vd, P=8, causal=True, layout=layout)
        got = (from_dev(got[0]), from_dev(got[1]))
    finally:
        ra.debug_set_delays(0, 0)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("zigzag", True)])
@pytest.mark.parametrize("delays", [(2000, 0), (0, 2000)])
def test_share_stream_order_under_delays(layout, causal, delays):
    import torch
    B, H, Hkv, N, d, P, rank = 1, 4, 4, 8 * 256, 128, 8, 5
    q, k, v = synth.qkv(22, B, H, Hkv, N, d, "bf16", Nq=N // P)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    kw = dict(P=P, rank=rank, causal=causal, layout=layout)
    ref = [from_dev(t) for t in ra.ring_attn_fwd_share(qd, kd, vd, **kw)]
    try:
        ra.debug_set_delays(*delays)
        got = [from_dev(t) for t in ra.ring_attn_fwd_share(qd, kd, vd, **kw)]
    finally:
        ra.debug_set_delays(0, 0)
    torch.cuda.synchronize()
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_fwd_ignores_stale_workspace(layout):
    """A workspace full of NaN bytes gives bitwise the same result as a zeroed one."""
    import torch
    B, H, Hkv, N, d, P = 1, 4, 4, 8 * 192, 128, 8
    qd, kd, vd = _inputs(23, B, H, Hkv, N, d)
    nb = ra.ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16)
    ws0 = torch.zeros(nb, dtype=torch.uint8, device="cuda:0")
    wsn = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda:0")
    a = [from_dev(t) for t in ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout, ws=ws0)]
    b = [from_dev(t) for t in ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout, ws=wsn)]
    assert np.all(np.isfinite(b[0]))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_step_state_checkpoint_resume():
    """Steps 0..3, state to the host and back through a cleared device, steps
    4..7: bitwise equal to the uninterrupted run."""
    import torch
    B, H, Hkv, Lq, d, P = 1, 4, 2, 256, 128, 8
    q, k, v = synth.qkv(24, B, H, Hkv, P * Lq, d, "bf16", Nq=Lq)
    qd = to_dev(q, "bf16")
    kb = [to_dev(np.ascontiguousarray(k[:, :, r * Lq:(r + 1) * Lq]), "bf16") for r in range(P)]
    vb = [to_dev(np.ascontiguousarray(v[:, :, r * Lq:(r + 1) * Lq]), "bf16") for r in range(P)]
    rank = 7
    order = [(rank - s) % P for s in range(P)]

    def run(blocks, state):
        for r in blocks:
            ra.ring_attn_step(qd, kb[r], vb[r], *state, causal=True, P=P, q_rank=rank, kv_rank=r)

    full = ra.init_state(B, H, Lq, d, "cuda:0")
    run(order, full)
    part = ra.init_state(B, H, Lq, d, "cuda:0")
    run(order[:4], part)
    saved = [t.cpu().numpy().copy() for t in part]
    for t in part:
        t.fill_(float("nan"))
    restored = [torch.from_numpy(x).to("cuda:0") for x in saved]
    run(order[4:], restored)
    for a, b in zip(full, restored):
        assert np.array_equal(from_dev(a), from_dev(b))
    out_full = [from_dev(t) for t in ra.ring_attn_finalize(*full)]
    out_res = [from_dev(t) for t in ra.ring_attn_finalize(*restored)]
    assert np.array_equal(out_full[0], out_res[0]) and np.array_equal(out_full[1], out_res[1])
