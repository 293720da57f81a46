"""Brute-force references used to pin the oracle (no tiles, no online softmax).

Each function is the textbook definition written directly on the full score
matrix, or a library routine (numpy softmax arithmetic, torch autograd in fp64
on the CPU).  None of it is shared with the oracle or the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch


def scores(q, k):
    """Full scaled score matrices per (b, h): [B, Hq, L, Lk] with GQA mapping."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    kk = np.repeat(k, G, axis=2)  # [B, Lk, Hq, d]
    return np.einsum("bihc,bjhc->bhij", q, kk) / np.sqrt(d)


def masked_attention(q, k, v, mask):
    """softmax over the keys where mask[b,h,i,j] is true, times V.

    Returns (o [B,L,Hq,d], lse [B,Hq,L]).  mask must leave every row non-empty.
    """
    B, L, Hq, d = q.shape
    G = Hq // k.shape[2]
    S = scores(q, k)
    Sm = np.where(mask, S, -np.inf)
    mx = Sm.max(axis=-1, keepdims=True)
    w = np.where(mask, np.exp(Sm - mx), 0.0)
    z = w.sum(axis=-1, keepdims=True)
    vv = np.repeat(v, G, axis=2)
    o = np.einsum("bhij,bjhc->bihc", w / z, vv)
    lse = (mx + np.log(z))[..., 0]
    return o, lse


def causal_mask(B, Hq, L):
    return np.broadcast_to(np.tril(np.ones((L, L), bool)), (B, Hq, L, L))


def dense_attention(q, k, v):
    B, L, Hq, d = q.shape
    return masked_attention(q, k, v, causal_mask(B, Hq, L))


def dense_probs(q, k):
    """Dense causal softmax probabilities [B, Hq, L, L]."""
    B, L, Hq, d = q.shape
    S = np.where(causal_mask(B, Hq, L), scores(q, k), -np.inf)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    return P / P.sum(axis=-1, keepdims=True)


def autograd_masked(q, k, v, dout, mask):
    """Gradients of sum(dout * o) for o = masked_attention(q, k, v, mask), via torch
    autograd in float64 on the CPU.  Also returns dL/dS (the gradient with
    respect to the scaled scores) for masking experiments."""
    B, L, Hq, d = q.shape
    G = Hq // k.shape[2]
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    tm = torch.tensor(np.ascontiguousarray(mask))
    kk = tk.repeat_interleave(G, dim=2)
    vv = tv.repeat_interleave(G, dim=2)
    S = torch.einsum("bihc,bjhc->bhij", tq, kk) / np.sqrt(d)
    S.retain_grad()
    P = torch.softmax(S.masked_fill(~tm, float("-inf")), dim=-1)
    o = torch.einsum("bhij,bjhc->bihc", P, vv)
    (o * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    return (tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(),
            S.grad.numpy(), P.detach().numpy())


def keep_to_keymask(keep, L, Bq, Bk):
    """Per-tile bitmap [B,Hq,nQB,nKT] (1 = kept) -> per-row key mask [B,Hq,L,L]
    restricted to legal causal keys."""
    B, Hq, nQB, nKT = keep.shape
    m = np.zeros((B, Hq, L, L), bool)
    kept = keep == 1
    for qb in range(nQB):
        for kt in range(nKT):
            sel = kept[:, :, qb, kt]
            if not sel.any():
                continue
            r0, r1 = qb * Bq, min(L, (qb + 1) * Bq)
            j0, j1 = kt * Bk, min(L, (kt + 1) * Bk)
            m[:, :, r0:r1, j0:j1] |= sel[:, :, None, None]
    return m & causal_mask(B, Hq, L)


def scores_to_qk(exp_scores):
    """Build (q, k) with d = L whose scaled scores are ln(exp_scores):
    k_j = one-hot(j), q_i = sqrt(d) ln(e_ij) (0 where e_ij <= 0)."""
    E = np.asarray(exp_scores, dtype=np.float64)
    L = E.shape[1]
    d = L
    with np.errstate(divide="ignore"):
        lnE = np.where(E > 0, np.log(np.where(E > 0, E, 1.0)), 0.0)
    q = (np.sqrt(d) * lnE).reshape(1, L, 1, d)
    k = np.eye(L).reshape(1, L, 1, d)
    return q, k
