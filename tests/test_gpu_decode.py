"""GPU parity of mala_decode (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import adaptive_tile_skipping_amd as mala
import mala_gen as G
from oracle import oracle_decode
from parity import bf16_tensor, compare_decisions, rel_l2_per_head, to_f64, unpack_bits

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
LSE_TOL = 1e-4


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def run_decode_case(di, tau, label=""):
    dev = _dev()
    B, Hq, d = di["q"].shape
    N, Hkv = di["k"].shape[1], di["k"].shape[2]
    nT = -(-N // 64)
    q, kc, vc = (bf16_tensor(di[x], dev) for x in ("q", "k", "v"))
    bits = torch.empty((B, Hkv, -(-nT // 32)), dtype=torch.int32, device=dev)
    print(f"[decode] {label} B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} tau={tau}", flush=True)
    o, lse, kept = mala.mala_decode(q, kc, vc, tau, decision_bits=bits)
    torch.cuda.synchronize()
    ref = oracle_decode(*(G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v")), tau, 64)
    gk = unpack_bits(bits.cpu().numpy(), nT)
    dec = compare_decisions(gk, ref["keep"], ref["margin"], descending=True)
    assert dec["nonexempt"] == 0, dec
    bad = (gk != ref["keep"]).any(-1)                     # [B, Hkv]
    Gq = Hq // Hkv
    badh = np.repeat(bad, Gq, axis=1)                      # [B, Hq]
    og = to_f64(o)
    # one slice per sequence: its output [Hq, d] (a single head's d-vector is too
    # few elements for a relative-L2 bound that includes the bf16 rounding of O)
    worst, glob = rel_l2_per_head(np.where(badh[..., None], 0.0, og)[:, None],
                                  np.where(badh[..., None], 0.0, ref["o"])[:, None], head_axis=1)
    assert worst <= O_TOL, (worst, glob)
    lg = lse.cpu().numpy().astype(np.float64)
    lerr = np.abs(lg - ref["lse"])[~badh]
    if lerr.size:
        assert lerr.max() <= LSE_TOL + 1e-5 * np.abs(ref["lse"]).max(), lerr.max()
    kt = kept.cpu().numpy()
    assert np.array_equal(kt[~bad], ref["kept_tiles"][~bad])
    assert np.array_equal(kt, gk.sum(-1))
    return dict(dec=dec, o_worst=worst, keep_frac=float(ref["keep"].mean()))


@pytest.mark.parametrize("N", [1, 63, 64, 65, 1000, 5000])
@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_decode_shapes(N, tau):
    di = G.decode_inputs(1000 + N, 3, N, 6, 2, 128)
    run_decode_case(di, tau, f"N={N}")


@pytest.mark.parametrize("Gq,Hkv,d", [(1, 2, 128), (16, 1, 128), (5, 1, 64), (8, 2, 64)])
def test_decode_groups(Gq, Hkv, d):
    di = G.decode_inputs(1100 + Gq, 2, 3000, Gq * Hkv, Hkv, d)
    for tau in (0.0, 1.0):
        run_decode_case(di, tau, f"G={Gq}")


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_decode_128k(tau):
    di = G.workload_inputs("decode_128k")
    print(run_decode_case(di, tau, "decode_128k"))


def test_decode_strided_cache():
    """The cache as a view with a padded head dimension."""
    dev = _dev()
    di = G.decode_inputs(1200, 2, 2000, 4, 2, 128)
    q, kc, vc = (bf16_tensor(di[x], dev) for x in ("q", "k", "v"))
    big = torch.zeros((2, 2000, 3, 128), dtype=torch.bfloat16, device=dev)
    kv = big[:, :, :2]
    kv.copy_(kc)
    bigv = torch.zeros_like(big)
    vv = bigv[:, :, :2]
    vv.copy_(vc)
    o1, l1, _ = mala.mala_decode(q, kv, vv, 1.0)
    o2, l2, _ = mala.mala_decode(q, kc, vc, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
