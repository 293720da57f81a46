"""Small numpy statement of MALA's rules -- TEST INFRASTRUCTURE ONLY.

Written separately from mala_oracle.c and used only to cross-check it on tiny
inputs (it materialises the full L x L score matrix per head).  The rule is
the one of "MassAlloc Attention: Let Attention Allocate Its Own Compute"
(page 2, "Forward: online sparse softmax" and "Backward: offline sparse
probabilities"; page 1, forward/backward paragraphs), with the same readings
as the C oracle: a row votes keep on an empty retained mass or when
exp(tile row max) / retained mass >= tau / L_i; the block keeps a tile when any
row votes; skipped tiles leave the state untouched; tiles are visited from the
diagonal toward earlier keys; backward keeps a tile when some row has
max_j exp(s_ij - LSE_i) >= tau / L_i.
"""
from __future__ import annotations

import numpy as np


def _log_thr(tau, Lvis):
    Lvis = np.asarray(Lvis, dtype=np.float64)
    if tau == 0:
        return np.full(Lvis.shape, -np.inf)
    return np.log(tau) - np.log(Lvis)


def rule_block(S, legal, Lvis, tau, tiles):
    """Apply the forward rule to one block of rows.

    S: [nr, n] scores (any value where illegal), legal: [nr, n] bool,
    Lvis: [nr] visible-key counts, tiles: list of (j0, j1) in visit order.
    Returns (weights [nr, n] of the retained keys (unnormalised, relative to
    the final row max), m [nr], l [nr], decisions list, margins list).
    """
    nr, n = S.shape
    th = _log_thr(tau, Lvis)
    m = np.full(nr, -np.inf)
    l = np.zeros(nr)
    kept_mask = np.zeros((nr, n), bool)
    decisions, margins = [], []
    for (j0, j1) in tiles:
        sl = np.where(legal[:, j0:j1], S[:, j0:j1], -np.inf)
        M = sl.max(axis=1)
        has = M > -np.inf
        with np.errstate(divide="ignore", invalid="ignore"):
            x = np.where(l == 0, np.inf, M - m - np.log(np.where(l > 0, l, 1.0)) - th)
        x = np.where(has, x, -np.inf)
        lam = x.max()
        keep = bool(lam >= 0)
        decisions.append(keep)
        margins.append(lam)
        if keep:
            mn = np.where(has, np.maximum(m, M), m)
            with np.errstate(invalid="ignore"):
                alpha = np.where(m == -np.inf, 0.0, np.exp(m - mn))
            p = np.where(legal[:, j0:j1], np.exp(sl - np.where(has, mn, 0.0)[:, None]), 0.0)
            l = np.where(has, l * alpha + p.sum(axis=1), l)
            m = mn
            kept_mask[:, j0:j1] |= legal[:, j0:j1]
    return kept_mask, m, l, decisions, margins


def fwd(q, k, v, tau, Bq, Bk):
    """q [B,L,Hq,d], k/v [B,L,Hkv,d] float64.  Returns o, lse, keep [B,Hq,nQB,nKT]
    (255 where not visited), kept_slots, omitted."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, L))
    keep = np.full((B, Hq, nQB, nKT), 255, np.uint8)
    margin = np.full((B, Hq, nQB, nKT), np.nan)
    slots = np.zeros((B, Hq, L), np.int32)
    omitted = np.zeros((B, Hq, L))
    causal = np.tril(np.ones((L, L), bool))
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            S = (q[b, :, h, :] @ k[b, :, kh, :].T) / np.sqrt(d)
            for qb in range(nQB):
                r0, r1 = qb * Bq, min(L, (qb + 1) * Bq)
                first = (r1 - 1) // Bk
                tiles = [(kt * Bk, min(L, (kt + 1) * Bk)) for kt in range(first, -1, -1)]
                Sb = S[r0:r1]
                leg = causal[r0:r1]
                kept, m, l, dec, mg = rule_block(Sb, leg, np.arange(r0, r1) + 1, tau, tiles)
                for t, kp, x in zip(range(first, -1, -1), dec, mg):
                    keep[b, h, qb, t] = kp
                    margin[b, h, qb, t] = x
                w = np.where(kept, np.exp(Sb - m[:, None]), 0.0)
                o[b, r0:r1, h, :] = (w @ v[b, :, kh, :]) / l[:, None]
                lse[b, h, r0:r1] = m + np.log(l)
                slots[b, h, r0:r1] = kept.sum(axis=1)
                # omitted probability mass among all legal keys
                zall = np.where(leg, np.exp(Sb - m[:, None]), 0.0).sum(axis=1)
                omitted[b, h, r0:r1] = 1.0 - l / zall
    return {"o": o, "lse": lse, "keep": keep, "margin": margin, "kept_slots": slots, "omitted": omitted}


def fwd_varlen(q, k, v, cu_q, cu_k, tau, Bq, Bk):
    """Packed sequences with the queries at the end of their keys: row i of a
    chunk of Lq queries over Lk keys sees keys j <= Lk - Lq + i, L_i = that
    count.  Key tiles start at key 0; query blocks at the chunk's first row.
    Returns o [Tq,Hq,d], lse [Hq,Tq], keep [B,Hq,nQB,nKT] (255 = not visited)."""
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    B = len(cu_q) - 1
    lqs = [cu_q[b + 1] - cu_q[b] for b in range(B)]
    lks = [cu_k[b + 1] - cu_k[b] for b in range(B)]
    nQB, nKT = max(1, -(-max(lqs) // Bq)), max(1, -(-max(lks) // Bk))
    o = np.zeros_like(q)
    lse = np.zeros((Hq, Tq))
    keep = np.full((B, Hq, nQB, nKT), 255, np.uint8)
    for b in range(B):
        Lq, Lk = lqs[b], lks[b]
        off = Lk - Lq
        qs, ks = cu_q[b], cu_k[b]
        vis = np.arange(Lk)[None, :] <= (off + np.arange(Lq))[:, None]     # [Lq, Lk]
        for h in range(Hq):
            kh = h // G
            S = (q[qs:qs + Lq, h, :] @ k[ks:ks + Lk, kh, :].T) / np.sqrt(d)
            for qb in range(-(-Lq // Bq)):
                r0, r1 = qb * Bq, min(Lq, (qb + 1) * Bq)
                first = (off + r1 - 1) // Bk
                tiles = [(kt * Bk, min(Lk, (kt + 1) * Bk)) for kt in range(first, -1, -1)]
                kept, m, l, dec, _ = rule_block(S[r0:r1], vis[r0:r1], off + np.arange(r0, r1) + 1, tau, tiles)
                for t, kp in zip(range(first, -1, -1), dec):
                    keep[b, h, qb, t] = kp
                w = np.where(kept, np.exp(S[r0:r1] - m[:, None]), 0.0)
                o[qs + r0:qs + r1, h, :] = (w @ v[ks:ks + Lk, kh, :]) / l[:, None]
                lse[h, qs + r0:qs + r1] = m + np.log(l)
    return {"o": o, "lse": lse, "keep": keep}


def bwd(q, k, v, o, dout, lse, tau, Bq, Bk):
    """Offline backward rule.  Returns dq, dk, dv, keep [B,Hq,nQB,nKT]."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    sc = 1.0 / np.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    keep = np.full((B, Hq, nQB, nKT), 255, np.uint8)
    margin = np.full((B, Hq, nQB, nKT), np.nan)
    causal = np.tril(np.ones((L, L), bool))
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            S = (q[b, :, h, :] @ k[b, :, kh, :].T) * sc
            th = _log_thr(tau, np.arange(L) + 1)
            P = np.where(causal, np.exp(S - lse[b, h][:, None]), 0.0)
            mask = np.zeros((L, L), bool)
            for qb in range(nQB):
                r0, r1 = qb * Bq, min(L, (qb + 1) * Bq)
                for kt in range(0, (r1 - 1) // Bk + 1):
                    j0, j1 = kt * Bk, min(L, (kt + 1) * Bk)
                    leg = causal[r0:r1, j0:j1]
                    x = np.where(leg, S[r0:r1, j0:j1] - lse[b, h, r0:r1, None] - th[r0:r1, None], -np.inf)
                    kp = bool(x.max() >= 0)
                    keep[b, h, qb, kt] = kp
                    margin[b, h, qb, kt] = x.max()
                    if kp:
                        mask[r0:r1, j0:j1] = leg
            Pm = np.where(mask, P, 0.0)
            D = (dout[b, :, h, :] * o[b, :, h, :]).sum(axis=1)
            dP = dout[b, :, h, :] @ v[b, :, kh, :].T
            dS = Pm * (dP - D[:, None])
            dq[b, :, h, :] = sc * dS @ k[b, :, kh, :]
            dk[b, :, kh, :] += sc * dS.T @ q[b, :, h, :]
            dv[b, :, kh, :] += Pm.T @ dout[b, :, h, :]
    return {"dq": dq, "dk": dk, "dv": dv, "keep": keep, "margin": margin}


def bwd_varlen(q, k, v, o, dout, lse, cu_q, cu_k, tau, Bq, Bk):
    """Offline backward rule over packed sequences (queries at the end of
    their keys; lse [Hq, Tq]).  Returns dq, dk, dv, keep [B,Hq,nQB,nKT]."""
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    B = len(cu_q) - 1
    lqs = [cu_q[b + 1] - cu_q[b] for b in range(B)]
    lks = [cu_k[b + 1] - cu_k[b] for b in range(B)]
    nQB, nKT = max(1, -(-max(lqs) // Bq)), max(1, -(-max(lks) // Bk))
    sc = 1.0 / np.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    keep = np.full((B, Hq, nQB, nKT), 255, np.uint8)
    for b in range(B):
        Lq, Lk = lqs[b], lks[b]
        off = Lk - Lq
        qs, ks = cu_q[b], cu_k[b]
        vis = np.arange(Lk)[None, :] <= (off + np.arange(Lq))[:, None]
        th = _log_thr(tau, off + np.arange(Lq) + 1)
        for h in range(Hq):
            kh = h // G
            Q, K, V = q[qs:qs + Lq, h], k[ks:ks + Lk, kh], v[ks:ks + Lk, kh]
            S = (Q @ K.T) * sc
            lz = lse[h, qs:qs + Lq]
            P = np.where(vis, np.exp(S - lz[:, None]), 0.0)
            mask = np.zeros((Lq, Lk), bool)
            for qb in range(-(-Lq // Bq)):
                r0, r1 = qb * Bq, min(Lq, (qb + 1) * Bq)
                for kt in range(0, (off + r1 - 1) // Bk + 1):
                    j0, j1 = kt * Bk, min(Lk, (kt + 1) * Bk)
                    leg = vis[r0:r1, j0:j1]
                    x = np.where(leg, S[r0:r1, j0:j1] - lz[r0:r1, None] - th[r0:r1, None], -np.inf)
                    kp = bool(x.max() >= 0)
                    keep[b, h, qb, kt] = kp
                    if kp:
                        mask[r0:r1, j0:j1] = leg
            Pm = np.where(mask, P, 0.0)
            Dr = (dout[qs:qs + Lq, h] * o[qs:qs + Lq, h]).sum(axis=1)
            dS = Pm * (dout[qs:qs + Lq, h] @ V.T - Dr[:, None])
            dq[qs:qs + Lq, h] = sc * dS @ K
            dk[ks:ks + Lk, kh] += sc * dS.T @ Q
            dv[ks:ks + Lk, kh] += Pm.T @ dout[qs:qs + Lq, h]
    return {"dq": dq, "dk": dk, "dv": dv, "keep": keep}


def decode(q, kc, vc, tau, Bkd):
    """q [B,Hq,d], caches [B,N,Hkv,d].  Returns o, lse, keep [B,Hkv,nT]."""
    B, Hq, d = q.shape
    N, Hkv = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    nT = -(-N // Bkd)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq))
    keep = np.zeros((B, Hkv, nT), np.uint8)
    margin = np.full((B, Hkv, nT), np.nan)
    for b in range(B):
        for kh in range(Hkv):
            S = (q[b, kh * G:(kh + 1) * G, :] @ kc[b, :, kh, :].T) / np.sqrt(d)
            tiles = [(t * Bkd, min(N, (t + 1) * Bkd)) for t in range(nT - 1, -1, -1)]
            kept, m, l, dec, mg = rule_block(S, np.ones_like(S, bool), np.full(G, N), tau, tiles)
            for t, kp, x in zip(range(nT - 1, -1, -1), dec, mg):
                keep[b, kh, t] = kp
                margin[b, kh, t] = x
            w = np.where(kept, np.exp(S - m[:, None]), 0.0)
            o[b, kh * G:(kh + 1) * G, :] = (w @ vc[b, :, kh, :]) / l[:, None]
            lse[b, kh * G:(kh + 1) * G] = m + np.log(l)
    return {"o": o, "lse": lse, "keep": keep, "margin": margin}


def per_key_row(exp_scores, tau):
    """One query row with Bq = Bk = 1, stated key by key in the pages' terms.

    `exp_scores[j]` = exp(s_j) for the row's visible keys 0..L-1 (L = len).
    Keys are visited from the newest (j = L-1) to the oldest; a key is kept
    when nothing is retained yet or when exp(s_j) / (retained mass) >= tau / L.
    Returns (kept index list in visit order, retained mass Z_R, omitted mass
    fraction Z_O / (Z_R + Z_O)).
    """
    e = [float(x) for x in exp_scores]
    L = len(e)
    Z = 0.0
    kept = []
    for j in range(L - 1, -1, -1):
        if Z == 0.0 or e[j] / Z >= tau / L:
            kept.append(j)
            Z += e[j]
    Zo = sum(e) - Z
    return kept, Z, Zo / (Z + Zo)
