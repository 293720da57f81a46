"""GPU parity of mala_bwd (through the C ABI) against the fp64 oracle.

The GPU backward consumes the GPU forward's O and LSE; the oracle backward
consumes the oracle forward's own O and LSE, so no value from the HIP path
reaches the oracle."""
import json

import numpy as np
import pytest
import torch

import adaptive_tile_skipping_amd as mala
import mala_gen as G
from oracle import oracle_bwd, oracle_fwd
from parity import (bf16_tensor, compare_decisions, forced_decisions, fp32_gradient_noise, grad_check,
                    rel_l2_per_head, to_f64, unpack_bits)

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-2


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _rows_of_blocks(blocks, B, Hq, L, Bq):
    nQB = -(-L // Bq)
    m = np.zeros((B, Hq, L), bool)
    for bid in blocks:
        bh, qb = divmod(bid, nQB)
        m[bh // Hq, bh % Hq, qb * Bq:min(L, qb * Bq + Bq)] = True
    return m


def run_bwd_case(inp, tau, Bq, Bk, qblocks=None, ktiles=None, label=""):
    """mala_bwd as a function of its inputs: both sides get the same (q, k, v, o,
    dout, lse), with o and lse taken from the oracle forward and rounded to the
    types the API stores (bf16 O, fp32 LSE).  Where the oracle forward was not
    run (sampled large cases), the GPU gets the GPU forward's O/LSE for rows no
    checked gradient depends on."""
    dev = _dev()
    B, L, Hq, d = inp["q"].shape
    Hkv = inp["k"].shape[2]
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    print(f"[bwd] {label} B={B} L={L} Hq={Hq} Hkv={Hkv} d={d} tau={tau}", flush=True)
    f64 = {x: G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")}
    fwd_blocks = None
    if qblocks is not None or ktiles is not None:
        need = set(qblocks or [])
        Gq = Hq // Hkv
        for kid in (ktiles or []):
            bk, kt = divmod(kid, nKT)
            b, kh = divmod(bk, Hkv)
            for g in range(Gq):
                for qb in range((kt * Bk) // Bq, nQB):
                    need.add((b * Hq + kh * Gq + g) * nQB + qb)
        fwd_blocks = sorted(need)
    rf = oracle_fwd(f64["q"], f64["k"], f64["v"], tau, Bq, Bk, blocks=fwd_blocks)
    o_bits = G.round_to_bf16_bits(np.nan_to_num(rf["o"]))
    lse32 = rf["lse"].astype(np.float32)
    o_in = bf16_tensor(o_bits, dev)
    lse_in = torch.from_numpy(lse32).to(dev)
    if fwd_blocks is not None:
        og, lg = mala.mala_fwd(q, k, v, tau, Bq, Bk)
        rows = torch.from_numpy(_rows_of_blocks(fwd_blocks, B, Hq, L, Bq)).to(dev)
        lse_in = torch.where(rows, lse_in, lg)
        o_in = torch.where(rows.permute(0, 2, 1)[..., None], o_in, og)
    bst = mala.make_stats(B, Hq, L, Bq, Bk, dev)
    dq, dk, dv = mala.mala_bwd(q, k, v, o_in, do, lse_in, tau, Bq, Bk, stats=bst)
    torch.cuda.synchronize()
    o_or = G.bf16_bits_to_f64(o_bits)
    rb = oracle_bwd(f64["q"], f64["k"], f64["v"], o_or, f64["dout"], lse32.astype(np.float64), tau, Bq, Bk,
                    qunits=qblocks, kunits=ktiles, cond=True)
    bkeep = unpack_bits(bst["decision_bits"].cpu().numpy(), nKT)
    # the backward's tiles do not depend on each other and both sides hold the
    # same O and LSE: each GPU decision is judged on its own (no cascades)
    dec = forced_decisions(np.where(rb["keep"] == 255, 255, bkeep), rb["keep"], rb["margin"])
    assert dec["nonexempt"] == 0, dec
    # rows touched by a (near-tie, exempt) decision mismatch are left out of the
    # gradient comparison: query rows of the block, key rows of the tile
    vis = rb["keep"] != 255
    mism = vis & (np.where(vis, bkeep, 0) != np.where(vis, rb["keep"], 0))
    qbad = np.zeros((B, L, Hq, 1), bool)
    kbad = np.zeros((B, L, Hkv, 1), bool)
    Gq = Hq // Hkv
    for b_, h_, qb_, kt_ in zip(*np.nonzero(mism)):
        qbad[b_, qb_ * Bq:(qb_ + 1) * Bq, h_] = True
        kbad[b_, kt_ * Bk:(kt_ + 1) * Bk, h_ // Gq] = True
    # binary32 noise of dP - D on the blocks whose gradients are compared
    nblocks = None
    if fwd_blocks is not None:
        nblocks = [(bid // nQB // Hq, bid // nQB % Hq, bid % nQB) for bid in fwd_blocks]
    ddq, ddk = fp32_gradient_noise(f64["q"], f64["k"], f64["v"], o_or, f64["dout"], lse32.astype(np.float64),
                                   rb["keep"], Bq, Bk, blocks=nblocks)
    res = check_grads({"dq": dq, "dk": dk, "dv": dv}, rb, {"dq": ddq, "dk": ddk}, qbad, kbad, label)
    if qblocks is None:
        kt_g = bst["kept_tiles"].cpu().numpy()
        clean_blk = ~mism.any(-1)
        assert np.array_equal(kt_g[clean_blk], (rb["keep"] == 1).sum(-1)[clean_blk])
        ks_g = bst["kept_slots"].cpu().numpy()
        ks_o = pins_keymask(rb["keep"], L, Bq, Bk).sum(-1)
        clean_rows = ~np.moveaxis(qbad[..., 0], 1, 2)
        assert np.array_equal(ks_g[clean_rows], ks_o[clean_rows])
    res["bwd_keep_frac"] = float((bkeep == 1).sum() / max(1, (rb["keep"] != 255).sum()))
    res["dec"] = dec
    return res


def check_grads(got, rb, noise, qbad, kbad, label="", heads=None):
    """grad_check of dq, dk, dv against the oracle (entries of rows and keys
    touched by an exempt decision left out; heads: optional q-head / KV-head
    index lists to restrict to).  Prints the raw errors and how many slices
    the binary32 noise term decided; asserts every slice passes."""
    res = {}
    for name in ("dq", "dk", "dv"):
        ref = rb[name]
        m = ~np.isnan(ref) & ~(qbad if name == "dq" else kbad)
        if heads is not None:
            hm = np.zeros(ref.shape[2], bool)
            hm[heads[0] if name == "dq" else heads[1]] = True
            m = m & hm[None, None, :, None]
        cond = rb.get(name + "_cond")
        res[name] = grad_check(to_f64(got[name]), np.nan_to_num(ref), None if cond is None else np.nan_to_num(cond),
                               noise.get(name), mask=m)
    print(f"grad check {label}:", {n: {x: (round(float(r[x]), 6) if isinstance(r[x], float) else r[x])
                                       for x in ("worst_raw", "global_raw", "slices", "floor_decided",
                                                 "worst_ratio", "err_over_noise", "noise_over_floor")}
                                   for n, r in res.items()}, flush=True)
    for name in ("dq", "dk", "dv"):
        assert res[name]["ok"], (name, res[name])
    return res


def pins_keymask(keep, L, Bq, Bk):
    import pins
    return pins.keep_to_keymask(keep, L, Bq, Bk)


def run_chain_case(inp, tau, Bq, Bk, diffuse_heads, label=""):
    """GPU forward -> GPU backward (the path mala_attention's autograd takes)
    against oracle forward -> oracle backward, the oracle's O and LSE rounded
    to the stored types (bf16, fp32) as the API stores them.  Checks the
    backward's decisions (forward mismatches count as cascades), that the GPU
    backward keeps no tile its own forward skipped, every gradient slice
    against tol |ref| + u |cond| (parity.grad_check), and the q heads in
    diffuse_heads (and their KV heads) against the plain 1e-2 relative
    tolerance."""
    dev = _dev()
    B, L, Hq, d = inp["q"].shape
    Hkv = inp["k"].shape[2]
    Gq = Hq // Hkv
    nKT = -(-L // Bk)
    print(f"[chain] {label} B={B} L={L} Hq={Hq} Hkv={Hkv} d={d} tau={tau}", flush=True)
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    fst = mala.make_stats(B, Hq, L, Bq, Bk, dev)
    o, lse = mala.mala_fwd(q, k, v, tau, Bq, Bk, stats=fst)
    bst = mala.make_stats(B, Hq, L, Bq, Bk, dev)
    dq, dk, dv = mala.mala_bwd(q, k, v, o, do, lse, tau, Bq, Bk, stats=bst)
    torch.cuda.synchronize()
    f64 = {x: G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")}
    rf = oracle_fwd(f64["q"], f64["k"], f64["v"], tau, Bq, Bk)
    o_or = G.bf16_bits_to_f64(G.round_to_bf16_bits(rf["o"]))
    lse_or = rf["lse"].astype(np.float32).astype(np.float64)
    rb = oracle_bwd(f64["q"], f64["k"], f64["v"], o_or, f64["dout"], lse_or, tau, Bq, Bk, cond=True)
    fkeep = unpack_bits(fst["decision_bits"].cpu().numpy(), nKT)
    bkeep = unpack_bits(bst["decision_bits"].cpu().numpy(), nKT)
    vis = rf["keep"] != 255
    fbad = (np.where(vis, fkeep, 0) != np.where(vis, rf["keep"], 0)).any(-1)
    dec = compare_decisions(np.where(vis, bkeep, 255), rb["keep"], rb["margin"], descending=False,
                            cascade_prefix=fbad)
    assert dec["nonexempt"] == 0, dec
    assert not np.any((bkeep == 1) & (fkeep == 0) & vis)
    # rows of blocks with any forward or backward decision mismatch, and keys
    # of their tiles, are left out
    mism = vis & ((np.where(vis, bkeep, 0) != np.where(vis, rb["keep"], 0)) | fbad[..., None])
    qbad = np.zeros((B, L, Hq, 1), bool)
    kbad = np.zeros((B, L, Hkv, 1), bool)
    for b_, h_, qb_, kt_ in zip(*np.nonzero(mism)):
        qbad[b_, qb_ * Bq:(qb_ + 1) * Bq, h_] = True
        kbad[b_, kt_ * Bk:(kt_ + 1) * Bk, h_ // Gq] = True
    ddq, ddk = fp32_gradient_noise(f64["q"], f64["k"], f64["v"], o_or, f64["dout"], lse_or, rb["keep"], Bq, Bk)
    got = {"dq": dq, "dk": dk, "dv": dv}
    res = check_grads(got, rb, {"dq": ddq, "dk": ddk}, qbad, kbad, label + " all heads")
    dkv = sorted({h // Gq for h in diffuse_heads})
    plain = check_grads(got, {n: rb[n] for n in ("dq", "dk", "dv")}, {}, qbad, kbad, label + " diffuse heads",
                        heads=(list(diffuse_heads), dkv))
    return dict(all=res, diffuse=plain, dec=dec)


def test_bwd_chain_fwd_to_bwd():
    inp = G.attn_inputs(950, 1, 1100, 4, 2, 128, 0.1, diffuse_kv_heads=(1,))
    run_chain_case(inp, 1.0, 128, 64, diffuse_heads=(2, 3), label="L=1100")


def test_bwd_chain_gqa_8k():
    """The matched-scale 8K case (16 q heads over 4 KV heads; KV heads 2-3,
    i.e. q heads 8-15, diffuse)."""
    w = G.WORKLOADS["gqa_8k"]
    print(run_chain_case(G.workload_inputs("gqa_8k"), 1.0, w["Bq"], w["Bk"], diffuse_heads=tuple(range(8, 16)),
                         label="gqa_8k"))


@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_bwd_tiny_512(tau):
    w = G.WORKLOADS["tiny_512"]
    print(run_bwd_case(G.workload_inputs("tiny_512"), tau, w["Bq"], w["Bk"], label="tiny_512"))


@pytest.mark.parametrize("L", [1, 77, 129, 1000])
@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_bwd_ragged_gqa(L, tau):
    inp = G.attn_inputs(700 + L, 2, L, 6, 2, 128, 0.1, diffuse_kv_heads=(1,))
    run_bwd_case(inp, tau, 128, 64, label=f"ragged L={L}")


@pytest.mark.parametrize("L", [900, 1000])
def test_bwd_dense_two_tile_form_ragged(L):
    """tau = 0 with enough (batch, KV head) x key-tile pairs for the two-key-tile
    dK/dV form: B * Hkv * ceil(nKT / 2) reaches the device's CU count.  The
    lengths end inside a query block and inside a key tile; L = 900 gives an odd
    number of key tiles (the last workgroup holds one), L = 1000 an even one.
    Diagonal and ragged steps take the masked path, the others the unmasked one."""
    B, Hq, Hkv = 4, 16, 8
    nKT = -(-L // 64)
    assert B * Hkv * ((nKT + 1) // 2) >= torch.cuda.get_device_properties(0).multi_processor_count
    inp = G.attn_inputs(870 + L, B, L, Hq, Hkv, 128, 0.1, diffuse_kv_heads=(2, 5))
    run_bwd_case(inp, 0.0, 128, 64, label=f"two-tile dense L={L}")


@pytest.mark.parametrize("L", [64, 200])
@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_bwd_d64(L, tau):
    inp = G.attn_inputs(800 + L, 1, L, 4, 2, 64, 0.2)
    run_bwd_case(inp, tau, 64, 64, label=f"d64 L={L}")


def test_bwd_gqa_8k():
    """The matched-scale 8K configuration, tau = 1; prints its parity record
    (decisions, raw and relative gradient errors per slice, kept tiles) as one
    JSON line."""
    w = G.WORKLOADS["gqa_8k"]
    r = run_bwd_case(G.workload_inputs("gqa_8k"), 1.0, w["Bq"], w["Bk"], label="gqa_8k")
    rec = {"parity_record": "gqa_8k backward, tau=1", "dec": r["dec"], "bwd_keep_frac": r["bwd_keep_frac"]}
    for n in ("dq", "dk", "dv"):
        rec[n] = {x: (float(r[n][x]) if isinstance(r[n][x], (float, np.floating)) else r[n][x])
                  for x in ("worst_raw", "global_raw", "slices", "floor_decided", "worst_ratio")}
    print(json.dumps(rec), flush=True)


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_bwd_train_128k_sampled(tau):
    """Full-size launch; dq checked on sampled query blocks, dk/dv on the last key
    tiles (at tau = 0 these are both tiles of one dK/dV workgroup and the first
    of the next)."""
    w = G.WORKLOADS["train_128k"]
    inp = G.workload_inputs("train_128k")
    nQB, nKT = 131072 // 128, 131072 // 64
    qblocks = [h * nQB + qb for h, qb in ((0, nQB - 1), (2, nQB - 1), (4, nQB - 2), (1, 700))]
    ktiles = [nKT - 1, nKT - 2, nKT - 3]
    print(run_bwd_case(inp, tau, w["Bq"], w["Bk"], qblocks=qblocks, ktiles=ktiles, label="train_128k sampled"))


def test_bwd_workspace_reuse_and_determinism_of_decisions():
    dev = _dev()
    inp = G.attn_inputs(900, 1, 1500, 4, 2, 128, 0.1)
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    o, lse = mala.mala_fwd(q, k, v, 1.0)
    ws = mala.bwd_workspace(1, 1500, 4, 2, 128, device=dev)
    s1 = mala.make_stats(1, 4, 1500, 128, 64, dev)
    s2 = mala.make_stats(1, 4, 1500, 128, 64, dev)
    g1 = mala.mala_bwd(q, k, v, o, do, lse, 1.0, ws=ws, stats=s1)
    g1 = [t.clone() for t in g1]
    g2 = mala.mala_bwd(q, k, v, o, do, lse, 1.0, ws=ws, stats=s2)
    torch.cuda.synchronize()
    assert torch.equal(s1["decision_bits"], s2["decision_bits"])
    # no atomics on any gradient: each is accumulated in registers and written once
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])


def test_bwd_scan_masks_future_keys_of_the_second_query_half():
    """Regression: on a diagonal key tile the decision must ignore every future
    key, including those pairing a wave's second 32 queries with the tile's
    second 32 keys.  Every query attends almost only to key 0; query 170 is
    also aligned with key 180, which it may not see.  No legal entry of key
    tile 2 reaches tau / L_i for query block 1, so the tile is skipped."""
    L, d = 256, 128
    rng = np.random.default_rng(7)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    wv = rng.standard_normal(d)
    wv -= (wv @ u) * u
    wv /= np.linalg.norm(wv)
    K = 0.1 * rng.standard_normal((L, d))
    K[0] = 16 * u
    K[180] = 16 * wv
    Q = np.tile(16 * u, (L, 1))
    Q[170] += 16 * wv
    V = rng.standard_normal((L, d))
    dO = rng.standard_normal((L, d))
    inp = {x: G.round_to_bf16_bits(a)[None, :, None, :] for x, a in (("q", Q), ("k", K), ("v", V), ("dout", dO))}
    r = run_bwd_case(inp, 1.0, 128, 64, label="masked future key")
    assert r["dec"]["mismatch"] == 0


def test_bwd_strided_views():
    """q/k/v as views into a packed [B, L, 3, H, d] buffer, o/dout into a
    [B, L, 2, H, d] one, and dq/dk/dv written into views of a [B, L, 3, H, d]
    output: the same gradients as contiguous tensors (B = 2, ragged L)."""
    dev = _dev()
    B, L, H, d = 2, 700, 4, 128
    inp = G.attn_inputs(510, B, L, H, H, d, 0.1)
    qkv = torch.stack([bf16_tensor(inp[x], dev) for x in ("q", "k", "v")], dim=2)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert not q.is_contiguous()
    o, lse = mala.mala_fwd(q.contiguous(), k.contiguous(), v.contiguous(), 1.0)
    od = torch.stack([o, bf16_tensor(inp["dout"], dev)], dim=2)
    o_v, do_v = od[:, :, 0], od[:, :, 1]
    out = torch.full((B, L, 3, H, d), float("nan"), dtype=torch.bfloat16, device=dev)
    g1 = mala.mala_bwd(q, k, v, o_v, do_v, lse, 1.0, dq=out[:, :, 0], dk=out[:, :, 1], dv=out[:, :, 2])
    g2 = mala.mala_bwd(q.contiguous(), k.contiguous(), v.contiguous(), o_v.contiguous(), do_v.contiguous(), lse, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])
    assert torch.isfinite(g1[0].float()).all()
