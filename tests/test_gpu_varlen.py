"""GPU parity of mala_fwd_varlen (packed variable-length batches, prefill onto
an existing cache) through the C ABI against the fp64 oracle."""
import numpy as np
import pytest
import torch

import adaptive_tile_skipping_amd as mala
import mala_gen as G
from oracle import oracle_fwd_varlen
from parity import bf16_tensor, compare_decisions, forced_decisions, rel_l2, to_f64, unpack_bits

pytestmark = pytest.mark.gpu

O_TOL = 2e-3       # max relative L2 error of O per slice (see _o_slices)
LSE_TOL = 1e-4
STAT_TOL = 0.01


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _o_slices(cu_q, Hq):
    """(row range, heads) of each O slice: one per (sequence, head), or one per
    sequence over all heads when it has fewer than 8 queries (a lone d-vector
    is too few elements for a bound that includes O's bf16 rounding)."""
    out = []
    for b in range(len(cu_q) - 1):
        r0, r1 = int(cu_q[b]), int(cu_q[b + 1])
        if r1 == r0:
            continue
        if r1 - r0 < 8:
            out.append((r0, r1, list(range(Hq))))
        else:
            out.extend((r0, r1, [h]) for h in range(Hq))
    return out


def run_varlen_case(inp, tau, Bq, Bk, blocks=None, stats_mode=True, label=""):
    dev = _dev()
    cu_q, cu_k = inp["cu_q"], inp["cu_k"]
    B = len(cu_q) - 1
    lq, lk = np.diff(cu_q), np.diff(cu_k)
    max_q, max_k = int(lq.max()), int(lk.max())
    Tq, Hq, d = inp["q"].shape
    Hkv = inp["k"].shape[1]
    q, k, v = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v"))
    cq = torch.from_numpy(cu_q).to(dev)
    ck = torch.from_numpy(cu_k).to(dev)
    st = mala.make_varlen_stats(B, Hq, Tq, max_q, max_k, Bq, Bk, dev, omitted=stats_mode)
    print(f"[fwd_varlen] {label} lens_q={lq.tolist()[:8]} lens_k={lk.tolist()[:8]} Hq={Hq} Hkv={Hkv} d={d} "
          f"tau={tau} Bq={Bq} Bk={Bk}", flush=True)
    o, lse = mala.mala_fwd_varlen(q, k, v, cq, ck, max_q, max_k, tau, Bq, Bk, stats=st)
    torch.cuda.synchronize()
    qf, kf, vf = (G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v"))
    ref = oracle_fwd_varlen(qf, kf, vf, cu_q, cu_k, tau, Bq, Bk, blocks=blocks)
    nQB, nKT = ref["keep"].shape[2], ref["keep"].shape[3]
    gkeep = unpack_bits(st["decision_bits"].cpu().numpy(), nKT)
    # blocks the comparison covers, and the query rows they own
    if blocks is None:
        sel = np.ones((B, Hq, nQB), bool)
    else:
        sel = np.zeros(B * Hq * nQB, bool)
        sel[np.asarray(blocks)] = True
        sel = sel.reshape(B, Hq, nQB)
    visited = np.array([[[qb * Bq < lq[b]] * 1 for qb in range(nQB)] for b in range(B)], bool)[:, None, :, 0]
    rows = np.zeros((Hq, Tq), bool)
    for b in range(B):
        for qb in range(nQB):
            r0, r1 = cu_q[b] + qb * Bq, min(cu_q[b + 1], cu_q[b] + qb * Bq + Bq)
            if r1 > r0:
                rows[:, r0:r1] = sel[b, :, qb, None]
    dec = compare_decisions(np.where(ref["keep"] == 255, 255, gkeep), ref["keep"], ref["margin"])
    if dec["mismatch"]:
        # teacher-forced replay of the GPU's decisions (see tests/parity.py)
        forced = np.where(ref["keep"] == 255, 255, gkeep).astype(np.uint8)
        ref = oracle_fwd_varlen(qf, kf, vf, cu_q, cu_k, tau, Bq, Bk, blocks=blocks, forced=forced)
        dec = dict(forced_decisions(np.where(ref["keep"] == 255, 255, gkeep), ref["keep"], ref["margin"]),
                   free_run=dec)
        ref["keep"] = np.where(ref["keep"] == 255, 255, gkeep).astype(np.uint8)   # the decisions followed
    assert dec["nonexempt"] == 0, dec
    # blocks past a sequence's queries: nothing visited, statistics zero
    kt_g = st["kept_tiles"].cpu().numpy()
    unv = ~np.broadcast_to(visited, (B, Hq, nQB))
    assert (kt_g[unv] == 0).all() and (gkeep[unv] == 0).all()
    bad = (np.where(ref["keep"] == 255, 0, gkeep) != np.where(ref["keep"] == 255, 0, ref["keep"])).any(-1)
    clean = rows.copy()
    for b in range(B):
        for qb in range(nQB):
            r0, r1 = cu_q[b] + qb * Bq, min(cu_q[b + 1], cu_q[b] + qb * Bq + Bq)
            if r1 > r0:
                clean[:, r0:r1] &= ~bad[b, :, qb, None]
    o_g, lse_g = to_f64(o), lse.cpu().numpy().astype(np.float64)
    worst = 0.0
    for r0, r1, hs in _o_slices(cu_q, Hq):
        m = rows[hs, r0:r1].T[..., None]                     # [rows, heads, 1]
        if not m.any():
            continue
        x = np.where(m, o_g[r0:r1][:, hs], 0.0)
        y = np.where(m, ref["o"][r0:r1][:, hs], 0.0)
        worst = max(worst, rel_l2(x, y))
    assert worst <= O_TOL, worst
    lerr = np.abs(lse_g - ref["lse"])[clean]
    if lerr.size:
        assert lerr.max() <= LSE_TOL + 1e-5 * np.abs(ref["lse"][clean]).max(), lerr.max()
    slots_g = st["kept_slots"].cpu().numpy()
    assert np.array_equal(slots_g[clean], ref["kept_slots"][clean])
    kt_o = (ref["keep"] == 1).sum(-1)
    assert np.array_equal(kt_g[sel & ~bad], kt_o[sel & ~bad])
    if stats_mode and rows.any():
        om_g = st["omitted_mass"].cpu().numpy().astype(np.float64)
        a, bb = om_g[rows].mean(), ref["omitted"][rows].mean()
        assert abs(a - bb) <= STAT_TOL * bb + 1e-9, (a, bb)
    return dict(dec=dec, o_worst=worst,
                keep_frac=float((ref["keep"] == 1).sum() / max(1, (ref["keep"] != 255).sum())))


@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_varlen_mix(tau):
    """Fresh prompts, chunks onto caches, a single token, an empty chunk."""
    w = G.WORKLOADS["varlen_mix"]
    inp = G.workload_inputs("varlen_mix")
    print(run_varlen_case(inp, tau, w["Bq"], w["Bk"], label="varlen_mix"))


@pytest.mark.parametrize("lens", [
    ((64, 1, 65, 130), (64, 200, 65, 777)),
    ((300, 5), (301, 1000)),
    ((0, 0, 3), (0, 10, 3)),
])
def test_varlen_d64(lens):
    inp = G.varlen_inputs(510, lens[0], lens[1], 4, 1, 64, 0.2)
    run_varlen_case(inp, 1.0, 64, 64, label="d64")


@pytest.mark.parametrize("off", [1, 63, 64, 100, 129])
def test_varlen_offsets(off):
    """Key offsets Lk - Lq that put the diagonal anywhere inside a key tile."""
    inp = G.varlen_inputs(520 + off, [200, 129], [200 + off, 129 + off], 6, 2, 128, 0.1, diffuse_kv_heads=(1,))
    run_varlen_case(inp, 1.0, 128, 64, label=f"off={off}")


def test_chunk_matches_full_forward_bitwise():
    """A chunk that starts at a multiple of Bq runs exactly the blocks, tiles and
    thresholds of the full forward over the same rows: identical bits."""
    dev = _dev()
    L, start = 3000, 1280
    full = G.attn_inputs(530, 1, L, 6, 2, 128, 0.1, diffuse_kv_heads=(1,))
    q, k, v = (bf16_tensor(full[x], dev) for x in ("q", "k", "v"))
    o_full, l_full = mala.mala_fwd(q, k, v, 1.0, 128, 64)
    cq = torch.tensor([0, L - start], dtype=torch.int32, device=dev)
    ck = torch.tensor([0, L], dtype=torch.int32, device=dev)
    o_c, l_c = mala.mala_fwd_varlen(q[0, start:].contiguous(), k[0], v[0], cq, ck, L - start, L, 1.0, 128, 64)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_full[0, start:])
    assert torch.equal(l_c, l_full[0][:, start:])


def test_varlen_equal_lengths_match_fixed_layout():
    """B sequences of one length L packed back to back equal the [B, L, H, d] call."""
    dev = _dev()
    inp = G.attn_inputs(540, 3, 700, 4, 2, 128, 0.1)
    q, k, v = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v"))
    o1, l1 = mala.mala_fwd(q, k, v, 1.0, 128, 64)
    cu = torch.arange(0, 4 * 700, 700, dtype=torch.int32, device=dev)
    o2, l2 = mala.mala_fwd_varlen(q.reshape(2100, 4, 128), k.reshape(2100, 2, 128), v.reshape(2100, 2, 128),
                                  cu, cu, 700, 700, 1.0, 128, 64)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1.reshape(2100, 4, 128))
    assert torch.equal(l2, l1.permute(1, 0, 2).reshape(4, 2100))


def test_varlen_skips_inconsistent_sequence():
    """A sequence whose lengths break Lq <= Lk is skipped by the kernels (its
    rows stay as they were); the others are computed as usual."""
    dev = _dev()
    inp = G.varlen_inputs(550, [100, 50], [300, 80], 4, 2, 128, 0.1)
    q, k, v = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v"))
    ok_o, ok_l = mala.mala_fwd_varlen(q, k, v, torch.from_numpy(inp["cu_q"]).to(dev),
                                      torch.from_numpy(inp["cu_k"]).to(dev), 100, 300, 1.0)
    # second sequence claims 50 queries over 20 keys
    cq = torch.tensor([0, 100, 150], dtype=torch.int32, device=dev)
    ck = torch.tensor([0, 300, 320], dtype=torch.int32, device=dev)
    o = torch.full_like(q, 7.0)
    lse = torch.full((4, 150), -3.0, device=dev)
    mala.mala_fwd_varlen(q, k[:320].contiguous(), v[:320].contiguous(), cq, ck, 100, 300, 1.0, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o[:100], ok_o[:100]) and torch.equal(lse[:, :100], ok_l[:, :100])
    assert (o[100:] == 7.0).all() and (lse[:, 100:] == -3.0).all()


def test_prefill_128k_sampled():
    """Full-size launch: the last 16K queries of the 128K training sequence onto
    the cache of the 112K keys before them; the oracle checks sampled blocks."""
    w = G.WORKLOADS["prefill_128k"]
    inp = G.workload_inputs("prefill_128k")
    nQB = 16384 // 128
    blocks = [h * nQB + qb for h, qb in ((0, 0), (1, 37), (2, 64), (3, nQB - 2), (4, nQB - 1))]
    print(run_varlen_case(inp, 1.0, w["Bq"], w["Bk"], blocks=blocks, stats_mode=False, label="prefill_128k"))


# ------------------------------------------------------------------ backward
from oracle import oracle_bwd_varlen  # noqa: E402
from parity import fp32_gradient_noise, grad_check  # noqa: E402


def run_bwd_varlen_case(inp, tau, Bq, Bk, label=""):
    """mala_bwd_varlen as a function of its inputs: both sides get the same
    (q, k, v, o, dout, lse), with o and lse from the oracle's varlen forward
    rounded to the stored types (bf16 O, fp32 LSE)."""
    dev = _dev()
    cu_q, cu_k = inp["cu_q"], inp["cu_k"]
    B = len(cu_q) - 1
    lq, lk = np.diff(cu_q), np.diff(cu_k)
    max_q, max_k = int(lq.max()), int(lk.max())
    Tq, Hq, d = inp["q"].shape
    Hkv = inp["k"].shape[1]
    Gq = Hq // Hkv
    print(f"[bwd_varlen] {label} lens_q={lq.tolist()[:8]} lens_k={lk.tolist()[:8]} Hq={Hq} Hkv={Hkv} d={d} "
          f"tau={tau}", flush=True)
    f64 = {x: G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")}
    rf = oracle_fwd_varlen(f64["q"], f64["k"], f64["v"], cu_q, cu_k, tau, Bq, Bk)
    o_bits = G.round_to_bf16_bits(np.nan_to_num(rf["o"]))
    lse32 = np.nan_to_num(rf["lse"]).astype(np.float32)
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    o_in = bf16_tensor(o_bits, dev)
    lse_in = torch.from_numpy(lse32).to(dev)
    cq, ck = torch.from_numpy(cu_q).to(dev), torch.from_numpy(cu_k).to(dev)
    bst = mala.make_varlen_stats(B, Hq, Tq, max_q, max_k, Bq, Bk, dev)
    dq, dk, dv = mala.mala_bwd_varlen(q, k, v, o_in, do, lse_in, cq, ck, max_q, max_k, tau, Bq, Bk, stats=bst)
    torch.cuda.synchronize()
    o64 = G.bf16_bits_to_f64(o_bits)
    rb = oracle_bwd_varlen(f64["q"], f64["k"], f64["v"], o64, f64["dout"],
                           lse32.astype(np.float64), cu_q, cu_k, tau, Bq, Bk, cond=True)
    nKT = rb["keep"].shape[3]
    bkeep = unpack_bits(bst["decision_bits"].cpu().numpy(), nKT)
    vis = rb["keep"] != 255
    assert (bkeep[~vis] == 0).all()
    # tiles of the backward do not depend on each other: each decision on its own
    dec = forced_decisions(np.where(vis, bkeep, 255), rb["keep"], rb["margin"])
    assert dec["nonexempt"] == 0, dec
    mism = vis & (np.where(vis, bkeep, 0) != np.where(vis, rb["keep"], 0))
    qbad = np.zeros((Tq, Hq), bool)
    kbad = np.zeros((inp["k"].shape[0], Hkv), bool)
    for b_, h_, qb_, kt_ in zip(*np.nonzero(mism)):
        qbad[cu_q[b_] + qb_ * Bq:min(cu_q[b_ + 1], cu_q[b_] + (qb_ + 1) * Bq), h_] = True
        kbad[cu_k[b_] + kt_ * Bk:min(cu_k[b_ + 1], cu_k[b_] + (kt_ + 1) * Bk), h_ // Gq] = True
    got = {n: to_f64(t) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))}
    worst = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    decided = {"dq": 0, "dk": 0, "dv": 0}
    for b in range(B):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if ke == ks:
            continue
        if qe == qs:
            # no query rows; the keys of such a sequence get exactly zero
            assert (got["dk"][ks:ke] == 0).all() and (got["dv"][ks:ke] == 0).all()
            continue
        # this sequence as a batch of one: [1, Lq, Hq, d], keys [1, Lk, Hkv, d]
        sq = {x: a[qs:qe][None] for x, a in (("q", f64["q"]), ("dout", f64["dout"]), ("o", o64))}
        sk = {x: f64[x][ks:ke][None] for x in ("k", "v")}
        lse_b = lse32[:, qs:qe].astype(np.float64)[None]
        keep_b = rb["keep"][b:b + 1]
        ddq, ddk = fp32_gradient_noise(sq["q"], sk["k"], sk["v"], sq["o"], sq["dout"], lse_b, keep_b, Bq, Bk,
                                       off=int((ke - ks) - (qe - qs)))
        for name, noise in (("dq", ddq), ("dk", ddk), ("dv", [])):
            sl = slice(qs, qe) if name == "dq" else slice(ks, ke)
            bad = (qbad if name == "dq" else kbad)[sl][None, ..., None]
            rep = grad_check(got[name][sl][None], rb[name][sl][None],
                             rb[name + "_cond"][sl][None] if name != "dv" else None, noise, mask=~bad)
            assert rep["ok"], (label, b, name, rep)
            worst[name] = max(worst[name], rep["worst_raw"])
            decided[name] += rep["floor_decided"]
    print("grad errors: worst raw per (sequence, head)", worst, "slices decided by the binary32 floor", decided,
          flush=True)
    clean = ~mism.any(-1)
    kt_g = bst["kept_tiles"].cpu().numpy()
    assert np.array_equal(kt_g[clean], (rb["keep"] == 1).sum(-1)[clean])
    return dict(dec=dec, worst=worst)


@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_bwd_varlen_mix(tau):
    w = G.WORKLOADS["varlen_mix"]
    inp = G.workload_inputs("varlen_mix")
    print(run_bwd_varlen_case(inp, tau, w["Bq"], w["Bk"], label="varlen_mix"))


@pytest.mark.parametrize("off", [1, 63, 100, 129])
@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_bwd_varlen_offsets(off, tau):
    inp = G.varlen_inputs(560 + off, [200, 129, 0], [200 + off, 129 + off, 50], 6, 2, 128, 0.1,
                          diffuse_kv_heads=(1,))
    run_bwd_varlen_case(inp, tau, 128, 64, label=f"off={off}")


def test_bwd_varlen_d64():
    inp = G.varlen_inputs(570, [64, 1, 65, 130], [64, 200, 65, 777], 4, 1, 64, 0.2)
    for tau in (0.0, 1.0):
        run_bwd_varlen_case(inp, tau, 64, 64, label="d64")


def test_bwd_chunk_matches_full_backward_bitwise():
    """With the full backward's own O / LSE rows, a chunk starting at a
    multiple of Bq gives the full backward's dq rows bit for bit."""
    dev = _dev()
    L, start = 3000, 1280
    full = G.attn_inputs(580, 1, L, 6, 2, 128, 0.1, diffuse_kv_heads=(1,))
    q, k, v, do = (bf16_tensor(full[x], dev) for x in ("q", "k", "v", "dout"))
    o, lse = mala.mala_fwd(q, k, v, 1.0, 128, 64)
    dq_f, _, _ = mala.mala_bwd(q, k, v, o, do, lse, 1.0, 128, 64)
    cq = torch.tensor([0, L - start], dtype=torch.int32, device=dev)
    ck = torch.tensor([0, L], dtype=torch.int32, device=dev)
    dq_c, _, _ = mala.mala_bwd_varlen(q[0, start:].contiguous(), k[0], v[0], o[0, start:].contiguous(),
                                      do[0, start:].contiguous(), lse[0][:, start:].contiguous(), cq, ck,
                                      L - start, L, 1.0, 128, 64)
    torch.cuda.synchronize()
    assert torch.equal(dq_c, dq_f[0, start:])


def test_bwd_varlen_equal_lengths_match_fixed_layout():
    dev = _dev()
    inp = G.attn_inputs(590, 3, 700, 4, 2, 128, 0.1)
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    for tau in (0.0, 1.0):
        o, lse = mala.mala_fwd(q, k, v, tau, 128, 64)
        g1 = mala.mala_bwd(q, k, v, o, do, lse, tau, 128, 64)
        cu = torch.arange(0, 4 * 700, 700, dtype=torch.int32, device=dev)
        pk = lambda x: x.reshape(2100, x.shape[2], 128)  # noqa: E731
        g2 = mala.mala_bwd_varlen(pk(q), pk(k), pk(v), pk(o), pk(do), lse.permute(1, 0, 2).reshape(4, 2100).contiguous(),
                                  cu, cu, 700, 700, tau, 128, 64)
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(pk(a), b)


def test_autograd_wrappers_match_direct_calls():
    """mala_attention / mala_attention_varlen: torch autograd reaches the same
    kernels as the direct forward and backward calls (identical bits)."""
    dev = _dev()
    inp = G.varlen_inputs(600, [300, 130], [300, 900], 4, 2, 128, 0.1)
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    cq, ck = (torch.from_numpy(inp[x]).to(dev) for x in ("cu_q", "cu_k"))
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = mala.mala_attention_varlen(qa, ka, va, cq, ck, 300, 900, 1.0)
    o.backward(do)
    o2, lse2 = mala.mala_fwd_varlen(q, k, v, cq, ck, 300, 900, 1.0)
    g2 = mala.mala_bwd_varlen(q, k, v, o2, do, lse2, cq, ck, 300, 900, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for a, b in zip((qa.grad, ka.grad, va.grad), g2):
        assert torch.equal(a, b)
    fi = G.attn_inputs(610, 1, 500, 4, 2, 128, 0.1)
    q, k, v, do = (bf16_tensor(fi[x], dev) for x in ("q", "k", "v", "dout"))
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    o = mala.mala_attention(qa, ka, va, 1.0)
    o.backward(do)
    o2, lse2 = mala.mala_fwd(q, k, v, 1.0)
    g2 = mala.mala_bwd(q, k, v, o2, do, lse2, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for a, b in zip((qa.grad, ka.grad, va.grad), g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("tau", [1.0, 0.0])
def test_varlen_many_ragged_sequences_fwd_bwd(tau):
    """40 sequences of random lengths (empty chunks, single tokens, chunks onto
    caches, fresh prompts) with 5 q heads per KV head.  At tau = 0 the 40 x 2
    (sequence, KV head) pairs x 4 key-tile pairs take the two-key-tile dK/dV
    form, whose steps meet diagonals shifted by the cache offsets."""
    rng = np.random.default_rng(620)
    lk = rng.integers(0, 400, size=40)
    lq = np.array([rng.integers(0, k + 1) if rng.random() < 0.7 else k for k in lk])
    lq[3], lk[3] = 1, 1
    lq[5] = 0
    inp = G.varlen_inputs(620, lq, lk, 10, 2, 128, 0.1, diffuse_kv_heads=(1,))
    print(run_varlen_case(inp, tau, 128, 64, label="40 ragged"))
    print(run_bwd_varlen_case(inp, tau, 128, 64, label="40 ragged"))


def test_varlen_larger_max_seqlen_changes_nothing():
    """max_seqlen_q / _k above the true maxima only add empty work units."""
    dev = _dev()
    inp = G.varlen_inputs(630, [200, 77], [300, 500], 4, 2, 128, 0.1)
    q, k, v, do = (bf16_tensor(inp[x], dev) for x in ("q", "k", "v", "dout"))
    cq, ck = (torch.from_numpy(inp[x]).to(dev) for x in ("cu_q", "cu_k"))
    o1, l1 = mala.mala_fwd_varlen(q, k, v, cq, ck, 200, 500, 1.0)
    o2, l2 = mala.mala_fwd_varlen(q, k, v, cq, ck, 277, 800, 1.0)
    g1 = mala.mala_bwd_varlen(q, k, v, o1, do, l1, cq, ck, 200, 500, 1.0)
    g2 = mala.mala_bwd_varlen(q, k, v, o1, do, l1, cq, ck, 277, 800, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
