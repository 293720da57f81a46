"""GPU parity over the context sweep (L = 1K .. 32K, 16 q heads over 4 KV heads,
half of them diffuse, tau in {0, 0.25, 1, 4}) and at extreme tolerances.

Long sequences are checked on sampled query blocks (forward, dQ) and key tiles
(dK, dV); the oracle never sees a value from the HIP path."""
import numpy as np
import pytest

import mala_gen as G
from test_gpu_bwd import run_bwd_case
from test_gpu_decode import run_decode_case
from test_gpu_fwd import run_fwd_case

pytestmark = pytest.mark.gpu

TAUS = [0.0, 0.25, 1.0, 4.0]


def _sample_blocks(Hq, nQB):
    heads = sorted({0, Hq // 3, Hq // 2 + 1, Hq - 1})
    qbs = sorted({0, nQB // 2, nQB - 1})
    return [h * nQB + qb for h in heads for qb in qbs]


@pytest.mark.parametrize("L", [1024, 2048, 4096, 8192, 16384, 32768])
@pytest.mark.parametrize("tau", TAUS)
def test_fwd_sweep(L, tau):
    w = G.WORKLOADS["sweep"]
    inp = G.workload_inputs("sweep", L=L, with_dout=False)
    nQB = -(-L // w["Bq"])
    blocks = None if L <= 2048 else _sample_blocks(w["Hq"], nQB)
    r = run_fwd_case(inp, tau, w["Bq"], w["Bk"], blocks=blocks, stats_mode=True, label=f"sweep L={L}")
    print(L, tau, r)


@pytest.mark.parametrize("L", [1024, 8192, 32768])
@pytest.mark.parametrize("tau", [0.25, 4.0])
def test_bwd_sweep(L, tau):
    w = G.WORKLOADS["sweep"]
    inp = G.workload_inputs("sweep", L=L)
    nQB, nKT = -(-L // w["Bq"]), -(-L // w["Bk"])
    if L <= 1024:
        r = run_bwd_case(inp, tau, w["Bq"], w["Bk"], label=f"sweep L={L}")
    else:
        qblocks = _sample_blocks(w["Hq"], nQB)
        ktiles = [kh * nKT + kt for kh in (0, w["Hkv"] - 1) for kt in (nKT - 1, nKT // 2)]
        r = run_bwd_case(inp, tau, w["Bq"], w["Bk"], qblocks=qblocks, ktiles=ktiles, label=f"sweep L={L}")
    print(L, tau, {k: v for k, v in r.items() if k != "dec"}, r["dec"])


@pytest.mark.parametrize("tau", [1e-6, 1e6])
def test_fwd_bwd_extreme_tau(tau):
    """Nearly dense (tiny tau) and nearly everything skipped but the first
    legal tiles (huge tau)."""
    inp = G.attn_inputs(1300, 2, 1000, 6, 2, 128, 0.1, diffuse_kv_heads=(1,))
    run_fwd_case(inp, tau, 128, 64, label=f"extreme tau={tau}")
    run_bwd_case(inp, tau, 128, 64, label=f"extreme tau={tau}")


@pytest.mark.parametrize("tau", [1e-38, 1e-6, 1e6, 1e30])
def test_decode_extreme_tau(tau):
    """tau / N outside and inside the linear-mass range of the decision pass."""
    di = G.decode_inputs(1400, 3, 5000, 6, 2, 128)
    run_decode_case(di, tau, f"extreme tau={tau}")
