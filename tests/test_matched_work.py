"""CPU checks of the matched-work allocation harness in bench.py (torch on the
CPU, small shapes): its tile reduction against direct sums, its omitted mass
for MALA's decisions against the oracle's, and the budget properties of the
three reference-mass policies."""
import numpy as np
import pytest
import torch

import bench
import mala_gen as G
from oracle import oracle_fwd

L, Hq, Hkv, d, Bq, Bk = 300, 4, 2, 16, 64, 32


def _inst(tag, tau=1.0):
    inp = G.attn_inputs(tag, 1, L, Hq, Hkv, d, 0.2, diffuse_kv_heads=(1,), with_dout=False)
    q, k, v = (G.bf16_bits_to_f64(inp[x])[0] for x in ("q", "k", "v"))
    mass, cost, o, evaluate = bench.dense_tile_stats(*(torch.from_numpy(x) for x in (q, k, v)), Bq, Bk)
    return q, k, v, mass, cost, o, evaluate


def test_tile_reduction_is_the_direct_sum():
    q, k, v, mass, cost, o, _ = _inst(800)
    for h in (0, 3):
        s = q[:, h] @ k[:, h // 2].T / np.sqrt(d)
        s = np.where(np.tril(np.ones((L, L), bool)), s, -np.inf)
        pr = np.exp(s - s.max(-1, keepdims=True))
        pr /= pr.sum(-1, keepdims=True)
        for qb, kt in ((0, 0), (2, 3), (4, 9), (4, 0)):
            r0, r1, j0, j1 = qb * Bq, min(L, qb * Bq + Bq), kt * Bk, min(L, kt * Bk + Bk)
            assert abs(float(mass[h, qb, kt]) - pr[r0:r1, j0:j1].sum()) <= 1e-12
            assert int(cost[h, qb, kt]) == int(np.tril(np.ones((L, L), bool))[r0:r1, j0:j1].sum())
        assert np.abs(o[:, h].numpy() - pr @ v[:, h // 2]).max() <= 1e-12


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
def test_omitted_mass_of_mala_decisions_matches_the_oracle(tau):
    """With the oracle's own keep bits as the policy, the harness's omitted
    mass per row is the oracle's omitted mass."""
    q, k, v, mass, cost, o, evaluate = _inst(801)
    r = oracle_fwd(q[None], k[None], v[None], tau, Bq, Bk)
    keep = torch.from_numpy(r["keep"][0] == 1)
    om, out = evaluate(keep)
    assert np.abs(om.numpy() - r["omitted"][0]).max() <= 1e-12
    assert np.abs(out.numpy() - r["o"][0]).max() <= 1e-10


def test_policies_spend_the_budget_and_keep_the_diagonal():
    q, k, v, mass, cost, o, evaluate = _inst(802)
    fz = bench.diagonal_tiles(cost, Bq, Bk, L)
    # every row has a legal key in the forced tiles
    om, out = evaluate(fz)
    assert torch.isfinite(out).all()
    total = int(0.4 * int(cost.sum()))
    ks = bench.alloc_within_blocks(mass, cost, bench.static_budget(cost, total, Bq, L), fz)
    ko = bench.alloc_global(mass, cost, total, fz)
    prof = torch.rand(cost.shape[:2], generator=torch.Generator().manual_seed(0), dtype=torch.float64)
    kh = bench.alloc_within_blocks(mass, cost, bench.profile_budget(prof, cost, total), fz)
    maxc = int(cost.max())
    for kp in (ks, ko, kh):
        assert (kp | ~fz).all()                       # forced tiles kept
        assert not (kp & (cost == 0)).any()           # nothing outside the causal range
        used = int((cost * kp).sum())
        assert used <= total
    # the global ranking leaves at most one tile of the budget unused
    assert total - int((cost * ko).sum()) < maxc
    # greedy by mass over the whole instance omits no more than the static split
    assert float(evaluate(ko)[0].sum()) <= float(evaluate(ks)[0].sum()) + 1e-12
    # static: every block gets the same slots per query, up to what it can use
    b = bench.static_budget(cost, total, Bq, L)
    rows = torch.tensor([min(Bq, L - i * Bq) for i in range(cost.shape[1])], dtype=torch.float64)
    per_q = b.double() / rows
    full = b < cost.sum(-1)
    assert float(per_q[full].max() - per_q[full].min()) <= 1.0
