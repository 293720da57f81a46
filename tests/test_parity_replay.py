"""CPU checks of the decision comparison the GPU tests use (tests/parity.py),
on decisions built from the oracle itself: a near-tie flip followed
consistently afterwards is one exempt mismatch and nothing else under the
teacher-forced replay, while decisions that ignore the flip's effect on the
retained state are caught (the side-by-side comparison of two free runs would
excuse them as cascades)."""
import math

import numpy as np

import mala_gen as G
from oracle import oracle_fwd
from parity import BAND, compare_decisions, forced_decisions

L, Hq, Hkv, d, Bq, Bk = 320, 4, 2, 32, 32, 32


def _inputs():
    inp = G.attn_inputs(905, 1, L, Hq, Hkv, d, 0.2, diffuse_kv_heads=(1,), with_dout=False)
    return tuple(G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v"))


def _near_tie_case():
    """tau and a block / tile where the tile's margin is +1e-4 (kept, inside
    the band) and skipping it changes a later decision of the block."""
    q, k, v = _inputs()
    base = oracle_fwd(q, k, v, 1.0, Bq, Bk)
    for idx in np.ndindex(*base["keep"].shape[:-1]):
        vis = np.nonzero(base["keep"][idx] != 255)[0][::-1]
        for t in vis[1:-1]:
            lam = base["margin"][idx + (t,)]
            if not (np.isfinite(lam) and 0.0 < lam < 20.0):
                continue
            tau = math.exp(lam - 1e-4)                   # shifts every margin by -(lam - 1e-4)
            r = oracle_fwd(q, k, v, tau, Bq, Bk)
            if not (0.0 < r["margin"][idx + (t,)] <= BAND and r["keep"][idx + (t,)] == 1):
                continue
            forced = np.full(r["keep"].shape, 255, np.uint8)
            forced[idx + (t,)] = 0
            f = oracle_fwd(q, k, v, tau, Bq, Bk, forced=forced)
            later = vis[vis < t]
            if (f["keep"][idx][later] != r["keep"][idx][later]).any():
                return q, k, v, tau, idx, t, r, f
    raise AssertionError("no near-tie tile whose flip changes a later decision")


def test_consistent_near_tie_flip_is_one_exempt_mismatch():
    q, k, v, tau, idx, t, r, f = _near_tie_case()
    gpu = np.where(r["keep"] == 255, 255, f["keep"]).astype(np.uint8)
    gpu[idx + (t,)] = 0                                  # the flip, then the rule from the new state
    rep = oracle_fwd(q, k, v, tau, Bq, Bk, forced=np.where(r["keep"] == 255, 255, gpu).astype(np.uint8))
    dec = forced_decisions(gpu, rep["keep"], rep["margin"])
    assert dec["mismatch"] == 1 and dec["exempt"] == 1 and dec["nonexempt"] == 0, dec
    free = compare_decisions(gpu, r["keep"], r["margin"])
    assert free["exempt"] == 1 and free["cascade"] >= 1 and free["nonexempt"] == 0, free


def test_decisions_that_ignore_the_flip_are_caught():
    q, k, v, tau, idx, t, r, f = _near_tie_case()
    gpu = r["keep"].copy()
    gpu[idx + (t,)] = 0                                  # flipped, but later decisions as if it had been kept
    free = compare_decisions(gpu, r["keep"], r["margin"])
    assert free["nonexempt"] == 0                        # side by side: a single exempt mismatch
    rep = oracle_fwd(q, k, v, tau, Bq, Bk, forced=np.where(r["keep"] == 255, 255, gpu).astype(np.uint8))
    dec = forced_decisions(gpu, rep["keep"], rep["margin"])
    assert dec["exempt"] >= 1 and dec["nonexempt"] >= 1, dec
