"""GPU parity of mala_fwd (through the C ABI) against the fp64 oracle."""
import json

import numpy as np
import pytest
import torch

import adaptive_tile_skipping_amd as mala
import mala_gen as G
from oracle import oracle_fwd
from parity import (bf16_tensor, compare_decisions, forced_decisions, rel_l2_per_head, to_f64, unpack_bits)

pytestmark = pytest.mark.gpu

O_TOL = 2e-3       # max relative L2 error of O per (b, h) slice
LSE_TOL = 1e-4     # |LSE_gpu - LSE_oracle| on rows of blocks without decision mismatch
STAT_TOL = 0.01    # relative difference of means (kept slots, omitted mass)


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def run_fwd_case(inp, tau, Bq, Bk, blocks=None, stats_mode=True, label=""):
    dev = _dev()
    B, L, Hq, d = inp["q"].shape
    Hkv = inp["k"].shape[2]
    q, k, v = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v"))
    st = mala.make_stats(B, Hq, L, Bq, Bk, dev, omitted=stats_mode)
    print(f"[fwd] {label} B={B} L={L} Hq={Hq} Hkv={Hkv} d={d} tau={tau} Bq={Bq} Bk={Bk}", flush=True)
    o, lse = mala.mala_fwd(q, k, v, tau, Bq, Bk, stats=st)
    torch.cuda.synchronize()
    qf, kf, vf = (G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v"))
    ref = oracle_fwd(qf, kf, vf, tau, Bq, Bk, blocks=blocks)
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    gkeep = unpack_bits(st["decision_bits"].cpu().numpy(), nKT)
    rows = np.zeros((B, Hq, L), bool)
    if blocks is None:
        sel = np.ones((B, Hq, nQB), bool)
    else:
        sel = np.zeros((B * Hq * nQB,), bool)
        sel[np.asarray(blocks)] = True
        sel = sel.reshape(B, Hq, nQB)
    for qb in range(nQB):
        rows[:, :, qb * Bq:min(L, qb * Bq + Bq)] = sel[:, :, qb, None]
    dec = compare_decisions(np.where(ref["keep"] == 255, 255, gkeep), ref["keep"], ref["margin"])
    if dec["mismatch"]:
        # teacher-forced replay: the oracle reruns every block following the
        # GPU's decisions, judges each one from that state, and its O, LSE and
        # statistics are those of the GPU's decisions, so every row is checked
        forced = np.where(ref["keep"] == 255, 255, gkeep).astype(np.uint8)
        ref = oracle_fwd(qf, kf, vf, tau, Bq, Bk, blocks=blocks, forced=forced)
        dec = dict(forced_decisions(np.where(ref["keep"] == 255, 255, gkeep), ref["keep"], ref["margin"]),
                   free_run=dec)
        ref["keep"] = np.where(ref["keep"] == 255, 255, gkeep).astype(np.uint8)   # the decisions followed
    assert dec["nonexempt"] == 0, dec
    # blocks whose decisions differ from the reference's are excluded from the
    # tight row checks (none after a replay)
    bad = (np.where(ref["keep"] == 255, 0, gkeep) != np.where(ref["keep"] == 255, 0, ref["keep"])).any(-1)
    clean_rows = rows.copy()
    for qb in range(nQB):
        clean_rows[:, :, qb * Bq:min(L, qb * Bq + Bq)] &= ~bad[:, :, qb, None]
    o_g, lse_g = to_f64(o), lse.cpu().numpy().astype(np.float64)
    # O: relative L2 per (b, h) over the selected rows
    msk = np.moveaxis(rows, 2, 1)[..., None]  # [B, L, Hq, 1]
    worst, glob = rel_l2_per_head(np.where(msk, o_g, 0.0), np.where(msk, ref["o"], 0.0))
    assert worst <= O_TOL, (worst, glob)
    lerr = np.abs(lse_g - ref["lse"])[clean_rows]
    if lerr.size:
        assert lerr.max() <= LSE_TOL + 1e-5 * np.abs(ref["lse"][clean_rows]).max(), lerr.max()
    slots_g = st["kept_slots"].cpu().numpy()
    assert np.array_equal(slots_g[clean_rows], ref["kept_slots"][clean_rows])
    ms_g, ms_o = slots_g[rows].mean(), ref["kept_slots"][rows].mean()
    assert abs(ms_g - ms_o) <= STAT_TOL * ms_o
    kt_g = st["kept_tiles"].cpu().numpy()
    kt_o = (ref["keep"] == 1).sum(-1)
    assert np.array_equal(kt_g[sel & ~bad], kt_o[sel & ~bad])
    res = dict(dec=dec, o_worst=float(worst), o_global=float(glob),
               keep_frac=float((ref["keep"] == 1).sum() / max(1, (ref["keep"] != 255).sum())),
               slots_per_query_gpu=float(ms_g), slots_per_query_oracle=float(ms_o))
    if stats_mode:
        om_g = st["omitted_mass"].cpu().numpy().astype(np.float64)
        a, bb = om_g[rows].mean(), ref["omitted"][rows].mean()
        assert abs(a - bb) <= STAT_TOL * bb + 1e-9, (a, bb)
        res.update(omitted_mean_gpu=float(a), omitted_mean_oracle=float(bb),
                   omitted_max_oracle=float(ref["omitted"][rows].max()))
    return res


@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_fwd_tiny_512(tau):
    w = G.WORKLOADS["tiny_512"]
    inp = G.workload_inputs("tiny_512")
    r = run_fwd_case(inp, tau, w["Bq"], w["Bk"], label="tiny_512")
    print(r)


@pytest.mark.parametrize("L", [1, 77, 128, 129, 1000])
@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_fwd_ragged_gqa(L, tau):
    inp = G.attn_inputs(300 + L, 2, L, 6, 2, 128, 0.1, diffuse_kv_heads=(1,))
    run_fwd_case(inp, tau, 128, 64, label=f"ragged L={L}")


@pytest.mark.parametrize("L", [64, 65, 300])
def test_fwd_d64_ragged(L):
    inp = G.attn_inputs(400 + L, 1, L, 4, 1, 64, 0.2)
    run_fwd_case(inp, 1.0, 64, 64, label=f"d64 L={L}")


def test_fwd_strided_views():
    """q/k/v as views into a packed [B, L, 3, H, d] buffer (non-contiguous heads)."""
    dev = _dev()
    inp = G.attn_inputs(500, 1, 520, 4, 4, 128, 0.1)
    qkv = torch.stack([bf16_tensor(inp[x], dev) for x in ("q", "k", "v")], dim=2)  # [B, L, 3, H, d]
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert not q.is_contiguous()
    o1, l1 = mala.mala_fwd(q, k, v, 1.0, 128, 64)
    o2, l2 = mala.mala_fwd(q.contiguous(), k.contiguous(), v.contiguous(), 1.0, 128, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_gqa_8k():
    """The matched-scale 8K configuration (B=1, Hq=16, Hkv=4, d=128, half the
    heads diffuse), tau = 1; prints its parity record as one JSON line."""
    w = G.WORKLOADS["gqa_8k"]
    inp = G.workload_inputs("gqa_8k", with_dout=False)
    r = run_fwd_case(inp, 1.0, w["Bq"], w["Bk"], label="gqa_8k")
    print(json.dumps({"parity_record": "gqa_8k forward, tau=1", **r}), flush=True)


@pytest.mark.parametrize("stats_mode", [False, True])
def test_fwd_train_128k_sampled(stats_mode):
    """Full-size launch (L = 131072, Hq = 5, Hkv = 1); the oracle checks 8
    query blocks of every head (40 of 5120).  Without statistics this is the
    launch the benchmark times; with them it also checks omitted mass."""
    w = G.WORKLOADS["train_128k"]
    inp = G.workload_inputs("train_128k", with_dout=False)
    nQB = 131072 // 128
    blocks = [h * nQB + qb for h in range(5) for qb in (0, 1, 129 + h, 517, 700 + 3 * h, 900, nQB - 2, nQB - 1)]
    r = run_fwd_case(inp, 1.0, w["Bq"], w["Bk"], blocks=blocks, stats_mode=stats_mode,
                     label=f"train_128k sampled stats={stats_mode}")
    print(r)


def test_fwd_deterministic():
    dev = _dev()
    inp = G.attn_inputs(600, 1, 2048, 4, 2, 128, 0.1)
    q, k, v = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v"))
    s1 = mala.make_stats(1, 4, 2048, 128, 64, dev)
    s2 = mala.make_stats(1, 4, 2048, 128, 64, dev)
    o1, l1 = mala.mala_fwd(q, k, v, 1.0, stats=s1)
    o2, l2 = mala.mala_fwd(q, k, v, 1.0, stats=s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(s1["decision_bits"], s2["decision_bits"])


def test_fwd_workspace_reused_across_shapes():
    """One workspace serves calls of different shapes in a row.  Each call's V
    copy re-zeroes the persistent kernel's work queues, so a smaller call after
    a larger one (and the larger one again) matches the oracle and a call on a
    fresh workspace bit for bit."""
    dev = _dev()
    big = G.attn_inputs(910, 2, 3000, 6, 2, 128, 0.1, diffuse_kv_heads=(1,))
    small = G.attn_inputs(911, 1, 700, 4, 1, 128, 0.2)
    ws = mala.fwd_workspace(2, 3000, 6, 2, 128, device=dev)
    qb, kb, vb = (bf16_tensor(big[x], dev) for x in ("q", "k", "v"))
    qs, ks, vs = (bf16_tensor(small[x], dev) for x in ("q", "k", "v"))
    print("[fwd] workspace reuse: B=2 L=3000, then B=1 L=700, then B=2 L=3000", flush=True)
    ob1, lb1 = mala.mala_fwd(qb, kb, vb, 1.0, ws=ws)
    os_, ls_ = mala.mala_fwd(qs, ks, vs, 1.0, ws=ws)
    ob2, lb2 = mala.mala_fwd(qb, kb, vb, 1.0, ws=ws)
    os_f, ls_f = mala.mala_fwd(qs, ks, vs, 1.0)          # its own workspace
    torch.cuda.synchronize()
    assert torch.equal(ob1, ob2) and torch.equal(lb1, lb2)
    assert torch.equal(os_, os_f) and torch.equal(ls_, ls_f)
    run_fwd_case(small, 1.0, 128, 64, label="small after big, own workspace")


def _v_as_fp16_rtz(v):
    """The forward's bf16 -> fp16 V conversion as documented: exact for
    2^-17 <= |v| <= 65504, truncated toward zero to a multiple of 2^-24 below
    2^-14 (fp16 subnormals), +-65504 above 65504."""
    a = np.minimum(np.abs(v), 65504.0)
    a = np.where(a < 2.0 ** -14, np.floor(a / 2.0 ** -24) * 2.0 ** -24, a)
    return np.sign(v) * a


@pytest.mark.parametrize("scale_exp", [16, -20])
def test_fwd_v_outside_fp16_range(scale_exp):
    """V scaled by 2^16 (a third of |v| above 65504) or 2^-20 (every |v| below
    2^-14): O equals the oracle's on V converted as the header documents, and
    differs from the oracle on the unconverted V where the conversion loses."""
    dev = _dev()
    inp = G.attn_inputs(620, 1, 600, 4, 2, 128, 0.1, diffuse_kv_heads=(1,), with_dout=False)
    qf, kf, vf = (G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v"))
    vs = vf * 2.0 ** scale_exp                       # exact: bf16 keeps fp32's exponent range
    vbits = G.round_to_bf16_bits(vs)
    assert np.array_equal(G.bf16_bits_to_f64(vbits), vs)
    conv = _v_as_fp16_rtz(vs)
    if scale_exp > 0:
        assert (np.abs(vs) > 65504).any()
    else:
        assert (np.abs(vs) < 2.0 ** -14).all() and (conv != vs).any()
    print(f"[fwd] V scaled by 2^{scale_exp} B=1 L=600 Hq=4 Hkv=2 d=128 tau=1", flush=True)
    q, k = (bf16_tensor(inp[x], dev) for x in ("q", "k"))
    v = bf16_tensor(vbits, dev)
    o, lse = mala.mala_fwd(q, k, v, 1.0, 128, 64)
    torch.cuda.synchronize()
    ref = oracle_fwd(qf, kf, conv, 1.0, 128, 64)
    worst, _ = rel_l2_per_head(to_f64(o), ref["o"])
    assert worst <= O_TOL, worst
    raw = oracle_fwd(qf, kf, vs, 1.0, 128, 64)
    worst_raw, _ = rel_l2_per_head(to_f64(o), raw["o"])
    print({"o_vs_converted_v": worst, "o_vs_unconverted_v": worst_raw}, flush=True)
    assert worst_raw > 10 * O_TOL
