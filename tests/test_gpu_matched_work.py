"""The matched-work allocation harness of bench.py on the GPU, against the
oracle (review page, "Performance validation: main results" -> "1) With equal
work, allocation is decisive", and the Table 1 caption: policies compared at
equal post-score work).

At a small size: MALA's kept set comes from the GPU forward's decision bits
and must match the oracle's decisions (exempt band aside); the harness, run in
fp64 on the GPU, must give the oracle's omitted mass and output for the
oracle's own kept set; the per-instance policy at MALA's budget must spend
that budget, agree with the same policy computed on the CPU from the oracle's
inputs, and omit no more mass than MALA (every tile it may choose has the same
cost, so taking tiles by mass is optimal for the budget).  One JSON line
reports the omitted mass of each policy."""
import json

import numpy as np
import pytest
import torch

import adaptive_tile_skipping_amd as mala
import bench
import mala_gen as G
from oracle import oracle_fwd
from parity import bf16_tensor, compare_decisions, unpack_bits

pytestmark = pytest.mark.gpu

L, Hq, Hkv, d, Bq, Bk = 1536, 4, 2, 128, 128, 64


@pytest.mark.parametrize("tau", [1.0, 16.0])
def test_matched_work_harness_on_gpu(tau):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dev = torch.device("cuda:0")
    inp = G.attn_inputs(720, 1, L, Hq, Hkv, d, 0.1, diffuse_kv_heads=(1,), with_dout=False)
    print(f"[matched_work] B=1 L={L} Hq={Hq} Hkv={Hkv} d={d} tau={tau}", flush=True)
    q, k, v = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v"))
    st = mala.make_stats(1, Hq, L, Bq, Bk, dev)
    mala.mala_fwd(q, k, v, tau, Bq, Bk, stats=st)
    torch.cuda.synchronize()
    nKT = -(-L // Bk)
    gkeep = unpack_bits(st["decision_bits"].cpu().numpy(), nKT)[0]          # [Hq, nQB, nKT]

    qf, kf, vf = (G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v"))
    ref = oracle_fwd(qf, kf, vf, tau, Bq, Bk)
    okeep = ref["keep"][0]
    dec = compare_decisions(np.where(okeep == 255, 255, gkeep), okeep, ref["margin"][0])
    assert dec["nonexempt"] == 0, dec

    # the harness in fp64 on the GPU (its fp64 matrix products there agree with
    # the CPU's to about 1e-7 of the output scale, not to 1e-15; the harness
    # reports percentages)
    mass, cost, o, evaluate = bench.dense_tile_stats(q[0].double(), k[0].double(), v[0].double(), Bq, Bk)
    ora_keep = torch.from_numpy(okeep == 1).to(dev)
    om, out = evaluate(ora_keep)
    assert np.abs(om.cpu().numpy() - ref["omitted"][0]).max() <= 1e-8
    assert np.abs(out.cpu().numpy() - ref["o"][0]).max() <= 1e-6 * np.abs(ref["o"][0]).max()

    mala_keep = torch.from_numpy(gkeep == 1).to(dev) & (cost > 0)
    fz = bench.diagonal_tiles(cost, Bq, Bk, L)
    assert bool((mala_keep | ~fz).all())                         # MALA keeps every diagonal tile
    budget = int((cost * mala_keep).sum())
    ko = bench.alloc_global(mass, cost, budget, fz)
    used = int((cost * ko).sum())
    assert budget - int(cost.max()) < used <= budget
    # every tile the policy may choose (legal, not forced) costs a full Bq x Bk
    assert bool((cost[(cost > 0) & ~fz] == Bq * Bk).all())
    om_o, _ = evaluate(ko)
    om_m, _ = evaluate(mala_keep)
    assert float(om_o.sum()) <= float(om_m.sum()) + 1e-9

    # the same policy from the oracle's inputs on the CPU
    mass_c, cost_c, _, evaluate_c = bench.dense_tile_stats(*(torch.from_numpy(x[0]) for x in (qf, kf, vf)), Bq, Bk)
    assert torch.equal(cost_c, cost.cpu())
    assert float((mass_c - mass.cpu()).abs().max()) <= 1e-7 * float(mass_c.max())
    ko_c = bench.alloc_global(mass_c, cost_c, budget, fz.cpu())
    om_c, _ = evaluate_c(ko_c)
    assert abs(float(om_c.sum()) - float(om_o.sum())) <= 1e-6 * max(1.0, float(om_o.sum()))

    ks = bench.alloc_within_blocks(mass, cost, bench.static_budget(cost, budget, Bq, L), fz)
    om_s, _ = evaluate(ks)
    rows = Hq * L
    print(json.dumps({"matched_work_gpu": {
        "tau": tau, "shape": f"B=1 L={L} Hq={Hq} Hkv={Hkv} d={d} Bq={Bq} Bk={Bk}",
        "slots_per_query": budget / rows, "decisions": dec,
        "omitted_mass_mean": {"mala": float(om_m.mean()), "per_instance_oracle": float(om_o.mean()),
                              "static": float(om_s.mean())}}}), flush=True)
