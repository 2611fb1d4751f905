"""GPU parity at the context lengths of the pages' scaling table: one kv head
plane of 9,437,184 tokens (2.4 GB per tensor in bf16, past 2 GiB), the size
of one device's share of a ring over such a sequence and of a long decode
cache ([TKG] title and §6 table: 4M- and 10M-token contexts).

  decode      B=1, H=4 / Hkv=1, L=9,437,184, d=128, P=8 ring blocks
  share       rank 7 of a P=8 causal ring over N=9,437,184 (H=1, d=128):
              its 1,179,648 queries against all keys, contiguous and striped
              (the striped plane is read through staged blocks)

The oracle (fp64) recomputes a seeded sample of query rows; rows are
independent, so the check is exact for those rows.
"""
import math
import time

import numpy as np
import pytest

import blockwise_ring_attention_attn_amd as ra
import oracle
import synth
from _util import assert_close, from_dev, host_vals, to_dev

pytestmark = pytest.mark.gpu

N, D, P, SEED = 9437184, 128, 8, 21


def _log(msg):
    print(f"\n[large] {msg}", flush=True)


@pytest.fixture(scope="module")
def kv():
    t0 = time.time()
    k = synth.tensor(SEED, synth.TENSOR_K, 1, 1, N, D, "bf16")
    v = synth.tensor(SEED, synth.TENSOR_V, 1, 1, N, D, "bf16")
    _log(f"k, v [1, 1, {N}, {D}] generated in {time.time() - t0:.1f} s")
    return k, v


@pytest.fixture(scope="module")
def kv_dev(kv):
    import torch
    k, v = kv
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    yield kd, vd
    del kd, vd
    torch.cuda.empty_cache()


def test_decode_9M_keys(kv, kv_dev):
    import torch
    kd, vd = kv_dev
    q = synth.tensor(SEED, synth.TENSOR_Q, 1, 4, 1, D, "bf16")
    _log(f"decode: H=4/Hkv=1 L={N} P={P}")
    out, lse = ra.ring_attn_decode(to_dev(q, "bf16"), kd, vd, P=P)
    torch.cuda.synchronize()
    k, v = kv
    Ow, Lw = oracle.decode(host_vals(q, "bf16"), host_vals(k, "bf16"), host_vals(v, "bf16"))
    eo, el = assert_close(from_dev(out), from_dev(lse), Ow, Lw[:, :, 0], "bf16", "decode 9M")
    _log(f"decode: max|dO|={eo:.2e} max|dlse|={el:.2e}")


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_share_9M_rank7(kv, kv_dev, layout):
    import torch
    kd, vd = kv_dev
    Bl = N // P
    rank = 7
    q = synth.tensor(SEED + 1, synth.TENSOR_Q, 1, 1, Bl, D, "bf16")
    _log(f"share {layout}: rank {rank}, {Bl} queries against {N} keys")
    t0 = time.time()
    out, lse = ra.ring_attn_fwd_share(to_dev(q, "bf16"), kd, vd, P=P, rank=rank, causal=True, layout=layout)
    torch.cuda.synchronize()
    _log(f"share {layout}: {time.time() - t0:.1f} s on the GPU")
    rows = np.unique(np.concatenate([[0, 1, Bl // 2, Bl - 2, Bl - 1],
                                     np.random.default_rng(SEED).integers(0, Bl, 11)]))
    rows_t = torch.from_numpy(rows).to(out.device)
    got_o, got_l = from_dev(out.index_select(2, rows_t)), from_dev(lse.index_select(2, rows_t))
    del out, lse
    qpos = oracle.host_positions(N, P, layout)[rank]
    k, v = kv
    Ow, Lw = oracle.attention(host_vals(q, "bf16"), host_vals(k, "bf16"), host_vals(v, "bf16"), causal=True,
                              scale=1 / math.sqrt(D), q_pos=qpos, rows=rows)
    eo, el = assert_close(got_o, got_l, Ow, Lw, "bf16", f"share 9M {layout}")
    _log(f"share {layout}: max|dO|={eo:.2e} max|dlse|={el:.2e} on {len(rows)} rows")
