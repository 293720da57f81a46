"""Pins of the variable-length / prefill forward of the fp64 oracle.

Reading (the summary page names prefill as a mode under the same tau; the
review page's "One tolerance governs everything" normalises by the row's
visible-key count): a chunk of Lq queries over Lk >= Lq keys holds the last Lq
positions of its sequence, so chunk row i sees keys j <= Lk - Lq + i and
L_i = Lk - Lq + i + 1.  Key tiles are aligned to key 0, query blocks to the
chunk's first row.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import mala_gen as G
from oracle import oracle_decode, oracle_fwd, oracle_fwd_varlen
from oracle import ref_numpy as R


def _f64(inp):
    return [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v")]


def _bottom_right_softmax(q, k, v, cu_q, cu_k):
    """Dense softmax attention with the bottom-right causal mask, in fp64."""
    Tq, Hq, d = q.shape
    Gq = Hq // k.shape[1]
    o = np.full(q.shape, np.nan)
    lse = np.full((Hq, Tq), np.nan)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        Lq, Lk = qe - qs, ke - ks
        vis = np.arange(Lk)[None, :] <= (Lk - Lq + np.arange(Lq))[:, None]
        for h in range(Hq):
            S = q[qs:qe, h] @ k[ks:ke, h // Gq].T / np.sqrt(d)
            S = np.where(vis, S, -np.inf)
            mx = S.max(-1, keepdims=True)
            w = np.exp(S - mx)
            o[qs:qe, h] = (w @ v[ks:ke, h // Gq]) / w.sum(-1, keepdims=True)
            lse[h, qs:qe] = mx[:, 0] + np.log(w.sum(-1))
    return o, lse


lens = st.lists(st.tuples(st.integers(0, 150), st.integers(0, 150)), min_size=1, max_size=4)


@settings(max_examples=50, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(lens, st.sampled_from([1, 8, 32, 64]), st.sampled_from([1, 16, 64]),
       st.sampled_from([0.0, 0.25, 1.0, 4.0]), st.integers(1, 2), st.integers(0, 10_000))
def test_varlen_c_oracle_matches_numpy(pairs, Bq, Bk, tau, Gq, seed):
    lq = [min(a, b) for a, b in pairs]
    lk = [max(a, b) for a, b in pairs]
    inp = G.varlen_inputs(300 + seed, lq, lk, 2 * Gq, 2, 8, 0.3, diffuse_kv_heads=(1,))
    q, k, v = _f64(inp)
    a = oracle_fwd_varlen(q, k, v, inp["cu_q"], inp["cu_k"], tau, Bq, Bk)
    b = R.fwd_varlen(q, k, v, inp["cu_q"], inp["cu_k"], tau, Bq, Bk)
    assert (a["keep"] == b["keep"]).all()
    if q.shape[0]:
        assert np.abs(a["o"] - b["o"]).max() <= 1e-11
        assert np.abs(a["lse"] - b["lse"]).max() <= 1e-11


@pytest.mark.parametrize("tiles", [(64, 64), (128, 64), (16, 32), (1, 1)])
def test_varlen_tau0_is_bottom_right_softmax(tiles):
    """tau = 0 keeps every tile: plain softmax attention with the queries at the
    end of their keys."""
    inp = G.varlen_inputs(310, [200, 1, 0, 77, 130], [200, 300, 50, 260, 131], 4, 2, 16, 0.2)
    q, k, v = _f64(inp)
    f = oracle_fwd_varlen(q, k, v, inp["cu_q"], inp["cu_k"], 0.0, *tiles)
    o, lse = _bottom_right_softmax(q, k, v, inp["cu_q"], inp["cu_k"])
    assert np.abs(f["o"] - o).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(f["lse"] - lse).max() <= 1e-12 * np.abs(lse).max()
    vis = f["keep"] != 255
    assert (f["keep"][vis] == 1).all()
    # every legal tile of every block is visited, nothing else
    cu_q, cu_k = inp["cu_q"], inp["cu_k"]
    Bq, Bk = tiles
    for b in range(len(cu_q) - 1):
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for qb in range(vis.shape[2]):
            r1 = min(Lq, (qb + 1) * Bq)
            n = (Lk - Lq + r1 - 1) // Bk + 1 if qb * Bq < Lq else 0
            assert vis[b, 0, qb].sum() == n


@settings(max_examples=30, deadline=None)
@given(st.integers(1, 40), st.integers(0, 60), st.sampled_from([0.25, 1.0, 4.0]), st.integers(0, 999))
def test_varlen_unit_tiles_match_key_by_key_statement(Lq, extra, tau, seed):
    """Bq = Bk = 1: each chunk row is decided alone, key by key from its newest
    visible key (Lk - Lq + i) down to key 0, with L = that row's key count."""
    Lk = Lq + extra
    inp = G.varlen_inputs(320 + seed, [Lq], [Lk], 1, 1, 8, 0.2)
    q, k, v = _f64(inp)
    f = oracle_fwd_varlen(q, k, v, inp["cu_q"], inp["cu_k"], tau, 1, 1)
    S = (q[:, 0, :] @ k[:, 0, :].T) / np.sqrt(8)
    for i in range(Lq):
        jl = Lk - Lq + i
        s = S[i, : jl + 1]
        kept, Z, _ = R.per_key_row(np.exp(s - s.max()), tau)
        got = np.nonzero(f["keep"][0, 0, i, : jl + 1] == 1)[0].tolist()
        assert sorted(kept) == got
        assert (f["keep"][0, 0, i, jl + 1:] == 255).all()
        assert abs(f["lse"][0, i] - (np.log(Z) + s.max())) <= 1e-12 * max(1, abs(s.max()))


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
@pytest.mark.parametrize("tiles,start", [((64, 64), 128), ((128, 64), 256), ((32, 16), 96)])
def test_chunk_at_block_boundary_reproduces_full_forward(tau, tiles, start):
    """A chunk whose first query sits at a multiple of Bq meets the same blocks,
    tiles and L_i as the full forward over the whole sequence, so its rows
    equal the full forward's rows from that position on."""
    L = 420
    Bq, Bk = tiles
    full = G.attn_inputs(330, 1, L, 4, 2, 16, 0.2, diffuse_kv_heads=(1,))
    fq, fk, fv = [G.bf16_bits_to_f64(full[x]) for x in ("q", "k", "v")]
    fr = oracle_fwd(fq, fk, fv, tau, Bq, Bk)
    cu_q = np.array([0, L - start], np.int32)
    cu_k = np.array([0, L], np.int32)
    cr = oracle_fwd_varlen(fq[0, start:], fk[0], fv[0], cu_q, cu_k, tau, Bq, Bk)
    assert np.array_equal(cr["o"], fr["o"][0, start:])
    assert np.array_equal(cr["lse"], fr["lse"][0][:, start:])
    nqb = cr["keep"].shape[2]
    assert np.array_equal(cr["keep"][0], fr["keep"][0][:, start // Bq:start // Bq + nqb])
    assert np.array_equal(cr["kept_slots"], fr["kept_slots"][0][:, start:])
    # and the generator draws the chunk as the tail of the same sequence
    ch = G.varlen_inputs(330, [L - start], [L], 4, 2, 16, 0.2, diffuse_kv_heads=(1,))
    assert np.array_equal(ch["q"], full["q"][0, start:]) and np.array_equal(ch["k"], full["k"][0])


@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_single_query_chunks_match_decode(tau):
    """Lq = 1 over an N-key cache with one q head per KV head (G = 1) is the
    decode rule: the same tiles newest first, L_i = N."""
    N, B, H, d = 700, 3, 2, 32
    di = G.decode_inputs(340, B, N, H, H, d)
    q, kc, vc = [G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v")]
    r = oracle_decode(q, kc, vc, tau, 64)
    cu_q = np.arange(B + 1, dtype=np.int32)
    cu_k = (np.arange(B + 1) * N).astype(np.int32)
    f = oracle_fwd_varlen(q, kc.reshape(B * N, H, d), vc.reshape(B * N, H, d), cu_q, cu_k, tau, 16, 64)
    assert np.array_equal(f["keep"][:, :, 0, :], r["keep"])
    assert np.abs(f["o"] - r["o"]).max() <= 1e-13 * np.abs(r["o"]).max()
    assert np.abs(f["lse"].T - r["lse"]).max() <= 1e-13 * np.abs(r["lse"]).max()
    assert np.abs(f["omitted"].T - r["omitted"]).max() <= 1e-12


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
def test_varlen_prop1_bound_and_first_tile(tau):
    """Omitted mass < tau / (1 + tau) per row, and each block keeps the tile of
    its rows' newest keys."""
    lq, lk = [300, 64, 1, 129], [300, 400, 999, 700]
    inp = G.varlen_inputs(350, lq, lk, 4, 2, 32, 0.3)
    q, k, v = _f64(inp)
    Bq, Bk = 64, 64
    f = oracle_fwd_varlen(q, k, v, inp["cu_q"], inp["cu_k"], tau, Bq, Bk)
    assert (f["omitted"] < tau / (1 + tau)).all()
    for b in range(len(lq)):
        for i in range(lq[b]):
            assert (f["keep"][b, :, i // Bq, (lk[b] - lq[b] + i) // Bk] == 1).all()
    # unvisited blocks of short sequences stay unvisited
    assert (f["keep"][2, :, 1:] == 255).all()


# ------------------------------------------------- decode with per-sequence cache lengths
@pytest.mark.parametrize("tau", [0.0, 0.25, 1.0, 4.0])
def test_decode_seqlens_match_one_row_varlen_forward(tau):
    """Decode with cache lengths N_b equals, for G = 1, the variable-length
    forward of one query over N_b keys (a separate code path): same tiles
    newest first, L_i = N_b, same retained set."""
    N, B, H, d = 500, 4, 3, 32
    lens = np.array([500, 1, 64, 333], np.int32)
    di = G.decode_inputs(360, B, N, H, H, d)
    q, kc, vc = [G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v")]
    r = oracle_decode(q, kc, vc, tau, 64, seqlens=lens)
    cu_q = np.arange(B + 1, dtype=np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kp = np.concatenate([kc[b, :lens[b]] for b in range(B)])
    vp = np.concatenate([vc[b, :lens[b]] for b in range(B)])
    f = oracle_fwd_varlen(q, kp, vp, cu_q, cu_k, tau, 16, 64)
    nT = r["keep"].shape[-1]
    assert np.array_equal(f["keep"][:, :, 0, :], r["keep"][..., :f["keep"].shape[-1]])
    for b in range(B):
        assert (r["keep"][b, :, -(-lens[b] // 64):nT] == 255).all()
    assert np.abs(f["o"] - r["o"]).max() <= 1e-13 * np.abs(r["o"]).max()
    assert np.abs(f["lse"].T - r["lse"]).max() <= 1e-13 * np.abs(r["lse"]).max()
    assert (r["kept_tiles"] == (r["keep"] == 1).sum(-1)).all()


def test_decode_seqlens_tau0_is_softmax_over_the_prefix():
    N, B, Hq, Hkv, d = 300, 3, 4, 2, 16
    lens = np.array([300, 17, 129], np.int32)
    di = G.decode_inputs(370, B, N, Hq, Hkv, d)
    q, kc, vc = [G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v")]
    r = oracle_decode(q, kc, vc, 0.0, 64, seqlens=lens)
    for b in range(B):
        for h in range(Hq):
            s = kc[b, :lens[b], h // 2] @ q[b, h] / np.sqrt(d)
            w = np.exp(s - s.max())
            o = w @ vc[b, :lens[b], h // 2] / w.sum()
            assert np.abs(r["o"][b, h] - o).max() <= 1e-12 * np.abs(o).max()
            assert abs(r["lse"][b, h] - (s.max() + np.log(w.sum()))) <= 1e-12 * max(1.0, abs(s.max()))


def test_decode_seqlens_full_length_is_plain_decode():
    di = G.decode_inputs(380, 2, 200, 4, 2, 16)
    q, kc, vc = [G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v")]
    a = oracle_decode(q, kc, vc, 1.0, 64)
    b = oracle_decode(q, kc, vc, 1.0, 64, seqlens=np.array([200, 200], np.int32))
    for key in ("o", "lse", "keep", "kept_tiles"):
        assert np.array_equal(a[key], b[key])
    with pytest.raises(ValueError):
        oracle_decode(q, kc, vc, 1.0, 64, seqlens=np.array([0, 200], np.int32))


# ------------------------------------------------- backward over packed sequences
from oracle import oracle_bwd, oracle_bwd_varlen  # noqa: E402


def _f64b(inp):
    return [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")]


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(lens, st.sampled_from([1, 8, 32, 64]), st.sampled_from([1, 16, 64]),
       st.sampled_from([0.0, 0.25, 1.0, 4.0]), st.integers(1, 2), st.integers(0, 10_000))
def test_varlen_backward_matches_numpy(pairs, Bq, Bk, tau, Gq, seed):
    lq = [min(a, b) for a, b in pairs]
    lk = [max(a, b) for a, b in pairs]
    inp = G.varlen_inputs(400 + seed, lq, lk, 2 * Gq, 2, 8, 0.3, diffuse_kv_heads=(1,))
    q, k, v, do = _f64b(inp)
    f = oracle_fwd_varlen(q, k, v, inp["cu_q"], inp["cu_k"], tau, Bq, Bk)
    a = oracle_bwd_varlen(q, k, v, f["o"], do, f["lse"], inp["cu_q"], inp["cu_k"], tau, Bq, Bk)
    b = R.bwd_varlen(q, k, v, f["o"], do, f["lse"], inp["cu_q"], inp["cu_k"], tau, Bq, Bk)
    assert (a["keep"] == b["keep"]).all()
    for n in ("dq", "dk", "dv"):
        if a[n].size:
            assert np.abs(a[n] - b[n]).max() <= 1e-10 * max(1.0, np.abs(b[n]).max()), n
    # nested support: the backward keeps no tile the forward skipped
    vis = b["keep"] != 255
    assert not ((b["keep"] == 1) & (f["keep"] == 0) & vis).any()


def test_varlen_backward_tau0_is_autograd():
    """tau = 0: the gradient of softmax attention with the queries at the end
    of their keys (torch autograd in fp64 on the CPU, per sequence)."""
    import torch
    lq, lk = [70, 1, 0, 33], [70, 90, 20, 100]
    inp = G.varlen_inputs(410, lq, lk, 4, 2, 16, 0.2)
    q, k, v, do = _f64b(inp)
    cu_q, cu_k = inp["cu_q"], inp["cu_k"]
    f = oracle_fwd_varlen(q, k, v, cu_q, cu_k, 0.0, 32, 16)
    r = oracle_bwd_varlen(q, k, v, f["o"], do, f["lse"], cu_q, cu_k, 0.0, 32, 16)
    for b in range(4):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        tq = torch.tensor(q[qs:qe], requires_grad=True)
        tk = torch.tensor(k[ks:ke], requires_grad=True)
        tv = torch.tensor(v[ks:ke], requires_grad=True)
        if qe > qs:
            S = torch.einsum("ihc,jhc->hij", tq, tk.repeat_interleave(2, dim=1)) / np.sqrt(16)
            vis = torch.arange(ke - ks)[None, :] <= (ke - ks - (qe - qs) + torch.arange(qe - qs))[:, None]
            P = torch.softmax(S.masked_fill(~vis, float("-inf")), dim=-1)
            o = torch.einsum("hij,jhc->ihc", P, tv.repeat_interleave(2, dim=1))
            (o * torch.tensor(do[qs:qe])).sum().backward()
            gq, gk, gv = tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()
        else:
            gq = np.zeros_like(q[qs:qe])
            gk, gv = np.zeros_like(k[ks:ke]), np.zeros_like(v[ks:ke])
        for name, got, ref in (("dq", r["dq"][qs:qe], gq), ("dk", r["dk"][ks:ke], gk), ("dv", r["dv"][ks:ke], gv)):
            if ref.size:
                assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), (b, name)


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
def test_varlen_backward_chunk_reproduces_full_dq(tau):
    """A chunk starting at a multiple of Bq: its dq rows and kept tiles equal the
    full backward's rows (its dk/dv hold only the chunk's queries' share)."""
    L, start, Bq, Bk = 300, 128, 64, 32
    full = G.attn_inputs(420, 1, L, 4, 2, 16, 0.2, diffuse_kv_heads=(1,))
    fq, fk, fv, fdo = [G.bf16_bits_to_f64(full[x]) for x in ("q", "k", "v", "dout")]
    ff = oracle_fwd(fq, fk, fv, tau, Bq, Bk)
    fb = oracle_bwd(fq, fk, fv, ff["o"], fdo, ff["lse"], tau, Bq, Bk)
    cu_q = np.array([0, L - start], np.int32)
    cu_k = np.array([0, L], np.int32)
    cb = oracle_bwd_varlen(fq[0, start:], fk[0], fv[0], ff["o"][0, start:], fdo[0, start:], ff["lse"][0][:, start:],
                           cu_q, cu_k, tau, Bq, Bk)
    assert np.array_equal(cb["dq"], fb["dq"][0, start:])
    nqb = cb["keep"].shape[2]
    assert np.array_equal(cb["keep"][0], fb["keep"][0][:, start // Bq:start // Bq + nqb])


def test_varlen_backward_equal_lengths_match_fixed_layout():
    B, L, Hq, Hkv, d = 3, 150, 4, 2, 16
    inp = G.attn_inputs(430, B, L, Hq, Hkv, d, 0.2)
    q, k, v, do = [G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")]
    f = oracle_fwd(q, k, v, 1.0, 64, 32)
    a = oracle_bwd(q, k, v, f["o"], do, f["lse"], 1.0, 64, 32)
    cu = np.arange(0, (B + 1) * L, L, dtype=np.int32)
    pk = lambda x: x.reshape(B * L, x.shape[2], d)  # noqa: E731
    r = oracle_bwd_varlen(pk(q), pk(k), pk(v), pk(f["o"]), pk(do), f["lse"].transpose(1, 0, 2).reshape(Hq, B * L),
                          cu, cu, 1.0, 64, 32)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(r[n], pk(a[n]))
    assert np.array_equal(r["keep"], a["keep"])


def test_varlen_backward_keys_without_queries_get_zero():
    inp = G.varlen_inputs(440, [0, 50], [40, 60], 2, 1, 16, 0.2)
    q, k, v, do = _f64b(inp)
    f = oracle_fwd_varlen(q, k, v, inp["cu_q"], inp["cu_k"], 1.0, 32, 16)
    r = oracle_bwd_varlen(q, k, v, f["o"], do, f["lse"], inp["cu_q"], inp["cu_k"], 1.0, 32, 16)
    assert (r["dk"][:40] == 0).all() and (r["dv"][:40] == 0).all()
    assert np.isfinite(r["dk"]).all() and np.isfinite(r["dq"]).all()
