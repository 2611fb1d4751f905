"""GPU tests of the ring driver's stream ordering, workspace hygiene and
resumable state (the step state between ring steps is a checkpoint), for the
forward ring, one device's share and the backward's reverse ring.

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


def _bwd_inputs(seed, B, H, Hkv, N, d, P, layout, dtype="bf16"):
    print(f"\n[driver bwd] seed={seed} B={B} H={H}/{Hkv} N={N} d={d} {dtype}", flush=True)
    q, k, v = synth.qkv(seed, B, H, Hkv, N, d, dtype)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    do = to_dev(synth.tensor(seed, synth.TENSOR_DOUT, B, H, N, d, dtype), dtype)
    out, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout)
    return qd, kd, vd, out, do, lse


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("delays", [(0, 0), (2000, 0), (0, 2000)])
def test_bwd_reverse_ring_staging(layout, delays):
    """The backward's reverse ring with its kv blocks staged on the copy
    stream (under injected delays on either stream) is bitwise the backward
    that reads every block in place."""
    args = _bwd_inputs(25, 1, 4, 2, 8 * 192, 128, 8, layout)
    kw = dict(P=8, causal=True, layout=layout)
    try:
        ra.debug_set_staging(False)
        ref = [from_dev(t) for t in ra.ring_attn_bwd(*args, **kw)]
        ra.debug_set_staging(True)
        ra.debug_set_delays(*delays)
        got = [from_dev(t) for t in ra.ring_attn_bwd(*args, **kw)]
    finally:
        ra.debug_set_staging(True)
        ra.debug_set_delays(0, 0)
    for a, b in zip(ref, got):
        assert np.all(np.isfinite(b)) and np.array_equal(a, b)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_bwd_ignores_stale_workspace(layout):
    """A backward workspace (staging buffers, accumulators, row statistics)
    full of NaN bytes gives bitwise the result of a zeroed one."""
    import torch
    B, H, Hkv, N, d, P = 1, 4, 2, 8 * 128, 64, 8
    args = _bwd_inputs(26, B, H, Hkv, N, d, P, layout)
    nb = ra.load().ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16)
    ws0 = torch.zeros(nb, dtype=torch.uint8, device="cuda:0")
    wsn = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda:0")
    a = [from_dev(t) for t in ra.ring_attn_bwd(*args, P=P, causal=True, layout=layout, ws=ws0)]
    b = [from_dev(t) for t in ra.ring_attn_bwd(*args, P=P, causal=True, layout=layout, ws=wsn)]
    for x, y in zip(a, b):
        assert np.all(np.isfinite(y)) and np.array_equal(x, y)


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_fwd_staged_equals_in_place(layout):
    """Forward ring and share with the exchange off (every block read in
    place) are bitwise the staged ones: the staging only moves bytes."""
    B, H, Hkv, N, d, P = 1, 4, 2, 8 * 256, 128, 8
    qd, kd, vd = _inputs(27, B, H, Hkv, N, d)
    try:
        ra.debug_set_staging(False)
        ref = [from_dev(t) for t in ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout)]
        ref_s = [from_dev(t) for t in ra.ring_attn_fwd_share(qd[:, :, :N // P].contiguous(), kd, vd, P=P, rank=3,
                                                             causal=True, layout=layout)]
    finally:
        ra.debug_set_staging(True)
    got = [from_dev(t) for t in ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout)]
    got_s = [from_dev(t) for t in ra.ring_attn_fwd_share(qd[:, :, :N // P].contiguous(), kd, vd, P=P, rank=3,
                                                         causal=True, layout=layout)]
    for a, b in zip(ref + ref_s, got + got_s):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("layout,delays", [("contiguous", (2000, 0)), ("zigzag", (0, 2000))])
def test_bwd_fp32_reverse_ring_staging(layout, delays):
    """The fp32 backward stages fp32 K and V blocks; staged under delays is
    bitwise the in-place backward."""
    args = _bwd_inputs(28, 1, 4, 2, 8 * 66, 64, 8, layout, "f32")
    kw = dict(P=8, causal=True, layout=layout)
    try:
        ra.debug_set_staging(False)
        ref = [from_dev(t) for t in ra.ring_attn_bwd(*args, **kw)]
        ra.debug_set_staging(True)
        ra.debug_set_delays(*delays)
        got = [from_dev(t) for t in ra.ring_attn_bwd(*args, **kw)]
    finally:
        ra.debug_set_staging(True)
        ra.debug_set_delays(0, 0)
    for a, b in zip(ref, got):
        assert np.all(np.isfinite(b)) and np.array_equal(a, b)


def test_bwd_fp32_ignores_stale_workspace():
    import torch
    B, H, Hkv, N, d, P = 1, 2, 1, 8 * 40, 128, 8
    args = _bwd_inputs(29, B, H, Hkv, N, d, P, "striped", "f32")
    nb = ra.load().ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_F32)
    ws0 = torch.zeros(nb, dtype=torch.uint8, device="cuda:0")
    wsn = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda:0")
    a = [from_dev(t) for t in ra.ring_attn_bwd(*args, P=P, causal=True, layout="striped", ws=ws0)]
    b = [from_dev(t) for t in ra.ring_attn_bwd(*args, P=P, causal=True, layout="striped", ws=wsn)]
    for x, y in zip(a, b):
        assert np.all(np.isfinite(y)) and np.array_equal(x, y)


def _bwd_share_inputs(seed, B, H, Hkv, N, d, P, rank, layout, dtype="bf16"):
    print(f"\n[driver bwd share] seed={seed} B={B} H={H}/{Hkv} N={N} d={d} rank={rank} {layout} {dtype}", flush=True)
    q, k, v = synth.qkv(seed, B, H, Hkv, N, d, dtype, Nq=N // P)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    do = to_dev(synth.tensor(seed, synth.TENSOR_DOUT, B, H, N // P, d, dtype), dtype)
    out, lse = ra.ring_attn_fwd_share(qd, kd, vd, P=P, rank=rank, causal=True, layout=layout)
    return qd, kd, vd, out, do, lse


@pytest.mark.parametrize("layout,rank,delays", [("contiguous", 7, (2000, 0)), ("contiguous", 4, (0, 2000)),
                                                ("striped", 2, (0, 2000)), ("zigzag", 5, (2000, 0))])
def test_bwd_share_staging(layout, rank, delays):
    """One device's share of the backward with its kv blocks staged on the
    copy stream (under injected delays on either stream) is bitwise the
    share that reads every block in place, and a workspace full of NaN
    bytes changes nothing."""
    import torch
    B, H, Hkv, N, d, P = 1, 4, 2, 8 * 192, 128, 8
    args = _bwd_share_inputs(32, B, H, Hkv, N, d, P, rank, layout)
    kw = dict(P=P, rank=rank, causal=True, layout=layout)
    try:
        ra.debug_set_staging(False)
        ref = [from_dev(t) for t in ra.ring_attn_bwd_share(*args, **kw)]
        ra.debug_set_staging(True)
        ra.debug_set_delays(*delays)
        got = [from_dev(t) for t in ra.ring_attn_bwd_share(*args, **kw)]
    finally:
        ra.debug_set_staging(True)
        ra.debug_set_delays(0, 0)
    nb = ra.load().ring_attn_bwd_share_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16)
    wsn = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda:0")
    stale = [from_dev(t) for t in ra.ring_attn_bwd_share(*args, **kw, ws=wsn)]
    for a, b, c in zip(ref, got, stale):
        assert np.all(np.isfinite(b)) and np.array_equal(a, b) and np.array_equal(a, c)


def test_bwd_share_fp32_staging():
    args = _bwd_share_inputs(33, 1, 2, 1, 8 * 40, 64, 8, 6, "striped", "f32")
    kw = dict(P=8, rank=6, causal=True, layout="striped")
    try:
        ra.debug_set_staging(False)
        ref = [from_dev(t) for t in ra.ring_attn_bwd_share(*args, **kw)]
        ra.debug_set_staging(True)
        ra.debug_set_delays(0, 2000)
        got = [from_dev(t) for t in ra.ring_attn_bwd_share(*args, **kw)]
    finally:
        ra.debug_set_staging(True)
        ra.debug_set_delays(0, 0)
    for a, b in zip(ref, got):
        assert np.all(np.isfinite(b)) and np.array_equal(a, b)


@pytest.mark.parametrize("op", ["fwd", "share", "bwd", "bwd_share", "bwd_steps", "decode"])
def test_graph_capture_replays(op):
    """The calls allocate nothing and order their two streams with events, so
    a caller can capture one into a HIP graph (the staging copies on the
    library's second stream join the capture through the fork event).  Each
    of three replays, with outputs overwritten by eager fills and the device
    synchronized in between, is bitwise the eager call."""
    import torch
    B, H, Hkv, N, d, P = 1, 4, 2, 8 * 256, 128, 8
    print(f"\n[graph] {op}", flush=True)
    q, k, v = synth.qkv(31, B, H, Hkv, N, d, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    dev = qd.device
    if op == "fwd":
        ws = torch.empty(ra.ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16), dtype=torch.uint8, device=dev)
        outs = (torch.empty_like(qd), torch.empty((B, H, N), dtype=torch.float32, device=dev))

        def call():
            ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout="striped", out=outs[0], lse=outs[1], ws=ws)
    elif op == "share":
        qs = qd[:, :, :N // P].contiguous()
        ws = torch.empty(ra.load().ring_attn_fwd_share_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16), dtype=torch.uint8,
                         device=dev)
        outs = (torch.empty_like(qs), torch.empty((B, H, N // P), dtype=torch.float32, device=dev))

        def call():
            ra.ring_attn_fwd_share(qs, kd, vd, P=P, rank=5, causal=True, layout="contiguous", out=outs[0],
                                   lse=outs[1], ws=ws)
    elif op == "bwd":
        do = to_dev(synth.tensor(31, synth.TENSOR_DOUT, B, H, N, d, "bf16"), "bf16")
        o, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout="zigzag")
        ws = torch.empty(ra.load().ring_attn_bwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16), dtype=torch.uint8,
                         device=dev)
        outs = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd))

        def call():
            ra.ring_attn_bwd(qd, kd, vd, o, do, lse, P=P, causal=True, layout="zigzag", dq=outs[0], dk=outs[1],
                             dv=outs[2], ws=ws)
    elif op == "bwd_share":
        qs = qd[:, :, :N // P].contiguous()
        do = to_dev(synth.tensor(31, synth.TENSOR_DOUT, B, H, N // P, d, "bf16"), "bf16")
        o, lse = ra.ring_attn_fwd_share(qs, kd, vd, P=P, rank=6, causal=True, layout="contiguous")
        ws = torch.empty(ra.load().ring_attn_bwd_share_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16),
                         dtype=torch.uint8, device=dev)
        outs = (torch.empty_like(qs), torch.empty_like(kd), torch.empty_like(vd))

        def call():
            ra.ring_attn_bwd_share(qs, kd, vd, o, do, lse, P=P, rank=6, causal=True, layout="contiguous",
                                   dq=outs[0], dk=outs[1], dv=outs[2], ws=ws)
    elif op == "bwd_steps":
        # a caller's own ring backward: prep per query block, the accumulators
        # cleared by fill kernels, then every (query block, kv block) step
        Bl = N // P
        do = to_dev(synth.tensor(31, synth.TENSOR_DOUT, B, H, N, d, "bf16"), "bf16")
        o, lse = ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout="contiguous")
        blk = lambda t, r: t[:, :, r * Bl:(r + 1) * Bl].contiguous()
        qs, os_, dos, ls = ([blk(t, r) for r in range(P)] for t in (qd, o, do, lse))
        ks, vs = [blk(kd, r) for r in range(P)], [blk(vd, r) for r in range(P)]
        rst = [torch.empty((B, H, Bl, 2), dtype=torch.float32, device=dev) for _ in range(P)]
        dq = [torch.empty((B, H, Bl, d), dtype=torch.float32, device=dev) for _ in range(P)]
        dk = [torch.empty((B, Hkv, Bl, d), dtype=torch.float32, device=dev) for _ in range(P)]
        dv = [torch.empty((B, Hkv, Bl, d), dtype=torch.float32, device=dev) for _ in range(P)]
        outs = tuple(rst + dq + dk + dv)

        def call():
            for t in dq + dk + dv:
                t.zero_()
            for r in range(P):
                ra.ring_attn_bwd_prep(os_[r], dos[r], ls[r], rowstat=rst[r])
            for s in range(P):
                for r in range(P):
                    j = (r + s) % P
                    ra.ring_attn_bwd_step(qs[r], ks[j], vs[j], dos[r], rst[r], dq[r], dk[j], dv[j], causal=True,
                                          P=P, q_rank=r, kv_rank=j)
    else:
        q1 = qd[:, :, :1].contiguous()
        ws = torch.empty(ra.ring_attn_decode_ws_bytes(B, H, Hkv, N, d, P), dtype=torch.uint8, device=dev)
        outs = (torch.empty_like(q1), torch.empty((B, H), dtype=torch.float32, device=dev))

        def call():
            ra.ring_attn_decode(q1, kd, vd, P=P, out=outs[0], lse=outs[1], ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()   # eager, on a side stream (the library sets up its per-device stream and events here)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [from_dev(t) for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [from_dev(t) for t in outs]
        for a, b in zip(ref, got):
            assert np.array_equal(a, b), f"{op}: replay {r} differs from the eager call"


def test_concurrent_calls_from_two_threads():
    """Two host threads, each with its own stream, inputs and workspace, run
    staged forward rings at the same time (ctypes releases the interpreter
    lock, so the enqueues interleave in the library; the per-device copy
    stream and its events are shared).  Every result is bitwise the one the
    same call gives alone."""
    import threading
    import torch
    B, H, Hkv, N, d, P = 1, 4, 2, 8 * 256, 128, 8
    cases = []
    for i, layout in enumerate(("contiguous", "striped")):
        q, k, v = synth.qkv(40 + i, B, H, Hkv, N, d, "bf16")
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        ref = [from_dev(t) for t in ra.ring_attn_fwd(qd, kd, vd, P=P, causal=True, layout=layout)]
        ws = torch.empty(ra.ring_attn_fwd_ws_bytes(B, H, Hkv, N, d, P, ra.RA_BF16), dtype=torch.uint8,
                         device=qd.device)
        cases.append(dict(q=qd, k=kd, v=vd, layout=layout, ref=ref, ws=ws, stream=torch.cuda.Stream(), got=[]))
    torch.cuda.synchronize()
    errors = []

    def work(c):
        try:
            with torch.cuda.stream(c["stream"]):
                for _ in range(4):
                    o, lse = ra.ring_attn_fwd(c["q"], c["k"], c["v"], P=P, causal=True, layout=c["layout"],
                                              ws=c["ws"], stream=c["stream"])
                    c["got"].append((o, lse))
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(c,)) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for c in cases:
        assert len(c["got"]) == 4
        for o, lse in c["got"]:
            assert np.array_equal(from_dev(o), c["ref"][0]) and np.array_equal(from_dev(lse), c["ref"][1])
