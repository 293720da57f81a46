"""Pins of the oracle's teacher-forced replay (oracle_fwd / oracle_fwd_varlen /
oracle_decode with `forced`), which the GPU tests use to judge each GPU
decision from the retained state the GPU itself had.

- Forcing the rule's own decisions reproduces the free run bit for bit.
- With one decision per block flipped, O and LSE are softmax attention
  restricted to the tiles the forced run kept (the forced tiles plus the
  rule's decisions elsewhere), by brute force on the full score matrix.
- The recorded margins are the rule's definition evaluated on that
  trajectory, written directly: at each tile, in visit order, a row's retained
  log-mass is the log-sum-exp of its legal scores in the earlier kept tiles,
  and the margin is the largest (tile row max - retained log-mass - theta_i)
  over rows with a legal key (+inf for a row with nothing retained), theta_i =
  ln tau - ln L_i (review page, "Forward: online sparse softmax").
- Tiles visited before the flipped one keep their decisions and margins.
"""
import numpy as np
import pytest

import mala_gen as G
import pins
from oracle import oracle_decode, oracle_fwd, oracle_fwd_varlen

L, Hq, Hkv, d, Bq, Bk = 320, 4, 2, 32, 64, 64


def _inputs(seed):
    inp = G.attn_inputs(seed, 1, L, Hq, Hkv, d, 0.2, diffuse_kv_heads=(1,), with_dout=False)
    return tuple(G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v"))


def _flip_second(keep):
    """forced array: the second visited tile of every block with at least two,
    flipped; 255 elsewhere.  Returns (forced, flipped tile per block or -1)."""
    forced = np.full(keep.shape, 255, np.uint8)
    at = np.full(keep.shape[:-1], -1, np.int64)
    for idx in np.ndindex(*keep.shape[:-1]):
        vis = np.nonzero(keep[idx] != 255)[0][::-1]          # visit order: newest tile first
        if len(vis) >= 2:
            t = vis[1]
            forced[idx + (t,)] = 1 - keep[idx + (t,)]
            at[idx] = t
    return forced, at


def _margins_by_definition(S, used, tau, Lvis, Bk):
    """Margins of one decision block from its score rows S [R, Lk] (-inf =
    illegal), the decisions followed `used` [nT] (255 = not visited), and each
    row's visible-key count Lvis [R]."""
    nT = used.shape[0]
    lam = np.full(nT, np.nan)
    theta = np.log(tau) - np.log(Lvis)
    kept_cols = np.zeros(S.shape[1], bool)
    for t in range(nT - 1, -1, -1):
        if used[t] == 255:
            continue
        cols = slice(t * Bk, min(S.shape[1], (t + 1) * Bk))
        best = -np.inf
        for r in range(S.shape[0]):
            tile = S[r, cols]
            if not np.isfinite(tile).any():
                continue                                       # no legal key: no vote
            prev = S[r, kept_cols]
            prev = prev[np.isfinite(prev)]
            if prev.size == 0:
                x = np.inf
            else:
                mx = prev.max()
                x = tile.max() - (mx + np.log(np.exp(prev - mx).sum())) - theta[r]
            best = max(best, x)
        lam[t] = best
        if used[t] == 1:
            kept_cols[cols] = True
    return lam


@pytest.mark.parametrize("tau", [0.25, 1.0, 4.0])
def test_forcing_own_decisions_reproduces_the_free_run(tau):
    q, k, v = _inputs(901)
    r = oracle_fwd(q, k, v, tau, Bq, Bk)
    f = oracle_fwd(q, k, v, tau, Bq, Bk, forced=r["keep"])
    for key in ("keep", "o", "lse", "kept_slots", "omitted"):
        assert np.array_equal(r[key], f[key], equal_nan=True), key
    assert np.array_equal(r["margin"], f["margin"], equal_nan=True)


@pytest.mark.parametrize("tau", [0.25, 1.0])
def test_forced_forward_follows_the_forced_decisions(tau):
    q, k, v = _inputs(902)
    r = oracle_fwd(q, k, v, tau, Bq, Bk)
    forced, at = _flip_second(r["keep"])
    assert (at >= 0).sum() >= 8
    f = oracle_fwd(q, k, v, tau, Bq, Bk, forced=forced)
    used = np.where(forced != 255, forced, f["keep"])
    used = np.where(f["keep"] == 255, 255, used)
    # O and LSE: softmax over the keys of the tiles followed
    o_ref, lse_ref = pins.masked_attention(q, k, v, pins.keep_to_keymask(used, L, Bq, Bk))
    assert np.abs(f["o"] - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())
    assert np.abs(f["lse"] - lse_ref).max() <= 1e-12 * max(1.0, np.abs(lse_ref).max())
    # margins and decisions on the forced trajectory, from the definition
    S = np.where(pins.causal_mask(1, Hq, L), pins.scores(q, k), -np.inf)[0]      # [Hq, L, L]
    for h in range(Hq):
        for qb in range(-(-L // Bq)):
            rows = np.arange(qb * Bq, min(L, (qb + 1) * Bq))
            lam = _margins_by_definition(S[h, rows], used[0, h, qb], tau, rows + 1.0, Bk)
            got = f["margin"][0, h, qb]
            vis = used[0, h, qb] != 255
            assert np.array_equal(np.isinf(lam[vis]), np.isinf(got[vis]))
            fin = vis & np.isfinite(lam)
            assert np.abs(lam[fin] - got[fin]).max(initial=0.0) <= 1e-9
            assert np.array_equal(f["keep"][0, h, qb][vis], (got[vis] >= 0).astype(np.uint8))
            # tiles visited before the flipped one are those of the free run
            t = at[0, h, qb]
            if t >= 0:
                before = np.arange(t + 1, used.shape[-1])
                assert np.array_equal(f["keep"][0, h, qb][before], r["keep"][0, h, qb][before])
                assert np.array_equal(f["margin"][0, h, qb][before], r["margin"][0, h, qb][before],
                                      equal_nan=True)


def test_forced_varlen_forward_matches_the_fixed_layout():
    """A packed batch of one full-length sequence replays exactly as the
    fixed-length forward under the same forcing."""
    q, k, v = _inputs(903)
    r = oracle_fwd(q, k, v, 1.0, Bq, Bk)
    forced, _ = _flip_second(r["keep"])
    f = oracle_fwd(q, k, v, 1.0, Bq, Bk, forced=forced)
    cu = np.array([0, L], np.int32)
    g = oracle_fwd_varlen(q[0], k[0], v[0], cu, cu, 1.0, Bq, Bk, forced=forced)
    assert np.array_equal(g["keep"], f["keep"])
    assert np.array_equal(g["margin"], f["margin"], equal_nan=True)
    assert np.array_equal(g["o"], f["o"][0])
    assert np.array_equal(g["lse"], f["lse"][0])


@pytest.mark.parametrize("tau", [0.25, 1.0])
def test_forced_decode(tau):
    B, N, Hqd, Hkvd, Bkd = 2, 700, 6, 2, 64
    di = G.decode_inputs(904, B, N, Hqd, Hkvd, d)
    q, kc, vc = (G.bf16_bits_to_f64(di[x]) for x in ("q", "k", "v"))
    r = oracle_decode(q, kc, vc, tau, Bkd)
    same = oracle_decode(q, kc, vc, tau, Bkd, forced=r["keep"])
    for key in ("keep", "o", "lse", "kept_tiles", "omitted"):
        assert np.array_equal(r[key], same[key], equal_nan=True), key
    forced, at = _flip_second(r["keep"])
    f = oracle_decode(q, kc, vc, tau, Bkd, forced=forced)
    used = np.where(forced != 255, forced, f["keep"])
    Gq = Hqd // Hkvd
    for b in range(B):
        for kh in range(Hkvd):
            keys = np.repeat(used[b, kh] == 1, Bkd)[:N]
            assert f["kept_tiles"][b, kh] == int((used[b, kh] == 1).sum())
            S = np.stack([kc[b, :, kh] @ q[b, kh * Gq + g] / np.sqrt(d) for g in range(Gq)])   # [G, N]
            for g in range(Gq):
                s = np.where(keys, S[g], -np.inf)
                mx = s.max()
                w = np.where(keys, np.exp(s - mx), 0.0)
                o_ref = (w / w.sum()) @ vc[b, :, kh]
                assert np.abs(f["o"][b, kh * Gq + g] - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())
                assert abs(f["lse"][b, kh * Gq + g] - (mx + np.log(w.sum()))) <= 1e-12 * max(1.0, abs(mx))
            lam = _margins_by_definition(S, used[b, kh], tau, np.full(Gq, float(N)), Bkd)
            got = f["margin"][b, kh]
            assert np.array_equal(np.isinf(lam), np.isinf(got))
            fin = np.isfinite(lam)
            assert np.abs(lam[fin] - got[fin]).max(initial=0.0) <= 1e-9
            t = at[b, kh]
            before = np.arange(t + 1, used.shape[-1])
            assert np.array_equal(f["keep"][b, kh][before], r["keep"][b, kh][before])
