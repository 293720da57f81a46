"""The forward, backward and decode launches captured in one HIP graph.

The library enqueues kernels only (no allocation, no memset: every buffer it
clears is cleared by its own kernels), so a caller can capture a whole step
and replay it.  Each replay, with unrelated eager work and synchronisations
between replays, must reproduce the eager results bit for bit."""
import numpy as np
import pytest
import torch

import adaptive_tile_skipping_amd as mala
import mala_gen as G
from parity import bf16_tensor

pytestmark = pytest.mark.gpu


def test_step_captured_in_a_graph_replays_exactly():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dev = torch.device("cuda:0")
    B, L, Hq, Hkv, d = 1, 2000, 6, 2, 128
    inp = G.attn_inputs(700, B, L, Hq, Hkv, d, 0.1, diffuse_kv_heads=(1,))
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    di = G.decode_inputs(701, 3, 3000, Hq, Hkv, d)
    qd, kc, vc = (bf16_tensor(di[x], dev) for x in ("q", "k", "v"))
    o, lse = torch.empty_like(q), torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    od, lsed = torch.empty_like(qd), torch.empty((3, Hq), dtype=torch.float32, device=dev)
    kept = torch.empty((3, Hkv), dtype=torch.int32, device=dev)
    fst = mala.make_stats(B, Hq, L, 128, 64, dev)
    fws = mala.fwd_workspace(B, L, Hq, Hkv, d, device=dev)
    bws = mala.bwd_workspace(B, L, Hq, Hkv, d, device=dev)
    dws = mala.decode_workspace(3, 3000, Hq, Hkv, d, 64, dev)
    outs = (o, lse, dq, dk, dv, od, lsed, kept, fst["decision_bits"], fst["kept_tiles"])

    def step():
        mala.mala_fwd(q, k, v, 1.0, o=o, lse=lse, stats=fst, ws=fws)
        mala.mala_bwd(q, k, v, o, do, lse, 1.0, dq=dq, dk=dk, dv=dv, ws=bws)
        mala.mala_decode(qd, kc, vc, 1.0, 64, o=od, lse=lsed, kept_tiles=kept, ws=dws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    other = torch.empty_like(q)
    for rep in range(4):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), rep
        # eager work between replays, on the same workspaces
        mala.mala_fwd(q, k, v, 4.0, o=other, ws=fws)
        mala.mala_decode(qd, kc, vc, 0.0, 64, ws=dws)
        torch.cuda.synchronize()
