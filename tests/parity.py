"""Comparison helpers for GPU-vs-oracle parity.

Decision parity: a GPU decision that differs from the oracle's is *exempt* when
the oracle's log-margin lies within ln(1 + 1e-3) of zero (the ratio is within
1e-3 relative of the threshold).  Once a block has an exempt mismatch, the two
runs no longer share the retained state, so the forward and decode tests then
rerun the oracle as a teacher-forced replay of the GPU's decisions
(forced_decisions): every GPU decision is judged from the GPU's own state, and
any disagreement outside the band fails.  compare_decisions (the free runs
side by side) counts later mismatches of such a block as *cascade*; it serves
the backward, whose tiles do not depend on each other.
"""
from __future__ import annotations

import math

import numpy as np

BAND = math.log1p(1e-3)


def unpack_bits(bits: np.ndarray, nKT: int) -> np.ndarray:
    """[..., nWords] int32/uint32 -> [..., nKT] uint8 (bit kt%32 of word kt/32)."""
    w = np.asarray(bits).astype(np.uint32)
    kt = np.arange(nKT)
    return ((w[..., kt // 32] >> (kt % 32).astype(np.uint32)) & 1).astype(np.uint8)


def compare_decisions(gpu_keep, ora_keep, ora_margin, descending: bool = True, cascade_prefix=None):
    """Compare per-tile decisions over the tiles the oracle visited.

    gpu_keep/ora_keep/ora_margin: [..., nT] (255 in ora_keep = not visited).
    descending: visit order is from the highest tile index to 0.
    cascade_prefix: optional boolean [...] array of blocks already perturbed
    upstream (e.g. forward blocks with a mismatch, for the backward): their
    mismatches count as cascade.
    Returns dict(total, mismatch, exempt, cascade, nonexempt, first_nonexempt).
    """
    gk = np.asarray(gpu_keep).astype(np.int64)
    ok = np.asarray(ora_keep).astype(np.int64)
    mg = np.asarray(ora_margin, dtype=np.float64)
    vis = ok != 255
    mism = vis & (gk != ok)
    out = dict(total=int(vis.sum()), mismatch=int(mism.sum()), exempt=0, cascade=0, nonexempt=0,
               first_nonexempt=None)
    if not mism.any():
        return out
    lead = mism.reshape(-1, mism.shape[-1])
    marg = mg.reshape(-1, mg.shape[-1])
    pre = None if cascade_prefix is None else np.asarray(cascade_prefix).reshape(-1)
    for r in np.nonzero(lead.any(axis=1))[0]:
        idx = np.nonzero(lead[r])[0]
        order = idx[::-1] if descending else idx
        perturbed = bool(pre[r]) if pre is not None else False
        for t in order:
            if perturbed:
                out["cascade"] += 1
            elif abs(marg[r, t]) <= BAND:
                out["exempt"] += 1
                perturbed = True
            else:
                out["nonexempt"] += 1
                if out["first_nonexempt"] is None:
                    out["first_nonexempt"] = (int(r), int(t), float(marg[r, t]))
                perturbed = True
    return out


def forced_decisions(gpu_keep, forced_keep, forced_margin):
    """Compare GPU decisions with the rule's own decisions in the oracle's
    teacher-forced replay of them (the oracle rerun following the GPU's
    decisions; forced_keep / forced_margin are its keep and margin).  Each GPU
    decision is judged from the retained state the GPU itself had, so every
    disagreement is the GPU's own: exempt when the oracle's margin there lies
    within the band, non-exempt otherwise.  Nothing is a cascade.
    Returns dict(total, mismatch, exempt, cascade=0, nonexempt, first_nonexempt).
    """
    gk = np.asarray(gpu_keep).astype(np.int64)
    ok = np.asarray(forced_keep).astype(np.int64)
    mg = np.asarray(forced_margin, dtype=np.float64)
    vis = ok != 255
    mism = vis & (gk != ok)
    ex = mism & (np.abs(mg) <= BAND)
    ne = mism & ~ex
    first = None
    if ne.any():
        idx = tuple(int(x) for x in np.argwhere(ne)[0])
        first = (idx, float(mg[idx]))
    return dict(total=int(vis.sum()), mismatch=int(mism.sum()), exempt=int(ex.sum()), cascade=0,
                nonexempt=int(ne.sum()), first_nonexempt=first)


def rel_l2(x: np.ndarray, y: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    n = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / n) if n > 0 else float(np.linalg.norm(x - y))


def rel_l2_per_head(x, y, head_axis: int = 2):
    """Max over (b, h) slices of the relative L2 error, and the global value."""
    x = np.moveaxis(np.asarray(x, np.float64), head_axis, 1)
    y = np.moveaxis(np.asarray(y, np.float64), head_axis, 1)
    norms = np.array([[np.linalg.norm(y[b, h]) for h in range(y.shape[1])] for b in range(y.shape[0])])
    worst = 0.0
    for b in range(x.shape[0]):
        for h in range(x.shape[1]):
            den = norms[b, h]
            err = np.linalg.norm(x[b, h] - y[b, h])
            worst = max(worst, err / den if den > 0 else err)
    return worst, rel_l2(x, y)


U32 = 2.0 ** -24


def gamma(n: int, u: float = U32) -> float:
    """gamma_n = n u / (1 - n u): the bound on the relative error of a sum of n
    terms in floating point with unit roundoff u, against the sum of their
    absolute values (Higham, "Accuracy and Stability of Numerical
    Algorithms", 2nd ed., section 3.1)."""
    return n * u / (1.0 - n * u)


def _tile_cols(keep_row, Lk, Bk, jmax):
    cols = [np.arange(kt * Bk, min((kt + 1) * Bk, Lk, jmax + 1)) for kt in np.nonzero(keep_row == 1)[0]
            if kt * Bk <= jmax]
    return np.concatenate(cols) if cols else np.zeros(0, np.int64)


def fp32_gradient_noise(q, k, v, o, dout, lse, keep, Bq, Bk, blocks=None, off: int = 0):
    """How far a binary32 evaluation of dP_ij = dO_i.v_j and D_i = dO_i.o_i
    moves dq and dk from their exact values (everything else exact).

    dS_ij = P_ij (dP_ij - D_i) subtracts the two dot products; on a row whose
    attention sits on one key (o_i = v_t) the exact difference cancels far
    below binary32 resolution, so no binary32 kernel can match such a row's
    exact dq (or the dk of that key) to a relative tolerance.  This returns,
    for two summation orders (a library float32 matrix product with pairwise
    sums; 16-term partial products summed in order, as a 16-deep matrix core
    accumulates), the gradient perturbation
        ddq_i = scale sum_j P_ij (err dP_ij - err D_i) k_j,
        ddk_j = scale sum_i P_ij (err dP_ij - err D_i) q_i,
    over the kept legal pairs, P_ij = exp(s_ij - lse_i) in fp64.

    q, o, dout [B, Lq, Hq, d]; k, v [B, Lk, Hkv, d]; lse [B, Hq, Lq]; keep
    [B, Hq, nQB, nKT] (1 = kept) -- the values both sides of a comparison get.
    Query rows see keys j <= off + i.  blocks: iterable of (b, h, qb) to
    evaluate (default all); dk entries only collect the evaluated blocks.
    Returns ([ddq_a, ddq_b], [ddk_a, ddk_b]) with the layouts of q and k."""
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    Gq = Hq // Hkv
    sc = 1.0 / np.sqrt(d)
    nQB = keep.shape[2]
    ddq = [np.zeros_like(q), np.zeros_like(q)]
    ddk = [np.zeros_like(k), np.zeros_like(k)]
    if blocks is None:
        blocks = [(b, h, qb) for b in range(B) for h in range(Hq) for qb in range(nQB)]
    for b, h, qb in blocks:
        r0, r1 = qb * Bq, min((qb + 1) * Bq, Lq)
        if r0 >= r1:
            continue
        kh = h // Gq
        cols = _tile_cols(keep[b, h, qb], Lk, Bk, off + r1 - 1)
        if cols.size == 0:
            continue
        Q, dO, O = q[b, r0:r1, h], dout[b, r0:r1, h], o[b, r0:r1, h]
        K, V = k[b, cols, kh], v[b, cols, kh]
        legal = cols[None, :] <= (off + np.arange(r0, r1))[:, None]
        S = sc * (Q @ K.T)
        P = np.where(legal, np.exp(np.where(legal, S, 0.0) - lse[b, h, r0:r1, None]), 0.0)
        dP = dO @ V.T
        D = (dO * O).sum(-1)
        dO32, V32, O32 = dO.astype(np.float32), V.astype(np.float32), O.astype(np.float32)
        # order a: library float32 product; pairwise float32 sums
        dPa = (dO32 @ V32.T).astype(np.float64)
        Da = np.sum(dO32 * O32, axis=-1, dtype=np.float32).astype(np.float64)
        # order b: dP from 16-term partial products accumulated in order; D
        # summed one product at a time from the last element down
        dPb = np.zeros(dP.shape, np.float32)
        for c0 in range(0, d, 16):
            dPb += dO32[:, c0:c0 + 16] @ V32[:, c0:c0 + 16].T
        prod = dO32 * O32
        Db = np.zeros(D.shape, np.float32)
        for c in range(d - 1, -1, -1):
            Db += prod[:, c]
        for x, (dPx, Dx) in enumerate(((dPa, Da), (dPb.astype(np.float64), Db.astype(np.float64)))):
            dS = P * ((dPx - dP) - (Dx - D)[:, None])
            ddq[x][b, r0:r1, h] += sc * (dS @ K)
            np.add.at(ddk[x][b, :, kh], cols, sc * (dS.T @ Q))
    return ddq, ddk


def grad_check(got, ref, cond, noise=None, mask=None, head_axis: int = 2, tol: float = 1e-2):
    """Per-(b, h) slice check of a gradient against the oracle.

    A slice passes when |got - ref| <= tol |ref| + u |cond|, u = 2^-24 and
    cond the oracle's dq_cond / dk_cond (None for dv, which has no
    cancellation).  gamma_d |cond| is the rigorous first-order bound on what
    binary32 evaluation of dP - D does to the slice; u |cond|, 1/d of it, is one
    unit roundoff of the same absolute sums.  Binary32 evaluations measured on
    these workloads stay near a tenth of it, so the floor admits a kernel
    whose dot products are ordinary binary32 sums and rejects any error about
    ten times that noise.  The floor only matters where the exact gradient
    cancels below binary32 resolution (a row attending to one key); elsewhere
    tol |ref| dominates.

    noise: optional measured binary32 perturbations (fp32_gradient_noise) for
    the report.  mask selects the compared entries (broadcast to got).

    Returns a report: worst raw relative error, global relative error, the
    number of slices, the number decided by the floor (raw relative error
    above tol), the largest |got - ref| / (tol |ref| + u |cond|), and with
    noise, the largest |got - ref| / |noise| over the floor-decided slices and
    the largest |noise| / (u |cond|)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.ones(got.shape, bool) if mask is None else np.broadcast_to(mask, got.shape)
    g = np.moveaxis(np.where(m, got, 0.0), head_axis, 1)
    r = np.moveaxis(np.where(m, ref, 0.0), head_axis, 1)
    cs = None if cond is None else np.moveaxis(np.where(m, np.asarray(cond, np.float64), 0.0), head_axis, 1)
    ns = None
    if noise:
        nmax = np.max([np.abs(np.where(m, n, 0.0)) for n in noise], axis=0)
        ns = np.moveaxis(nmax, head_axis, 1)
    rep = dict(slices=0, floor_decided=0, worst_raw=0.0, worst_ratio=0.0, err_over_noise=0.0,
               noise_over_floor=0.0, global_raw=rel_l2(np.where(m, got, 0.0), np.where(m, ref, 0.0)))
    for b in range(g.shape[0]):
        for h in range(g.shape[1]):
            rn = np.linalg.norm(r[b, h])
            en = np.linalg.norm(g[b, h] - r[b, h])
            if rn == 0 and en == 0:
                continue
            rep["slices"] += 1
            floor = U32 * np.linalg.norm(cs[b, h]) if cs is not None else 0.0
            raw = en / rn if rn > 0 else np.inf
            rep["worst_raw"] = max(rep["worst_raw"], raw)
            allow = tol * rn + floor
            rep["worst_ratio"] = max(rep["worst_ratio"], en / allow if allow > 0 else np.inf)
            if raw > tol:
                rep["floor_decided"] += 1
            if ns is not None and floor > 0:
                nz = np.linalg.norm(ns[b, h])
                rep["noise_over_floor"] = max(rep["noise_over_floor"], nz / floor)
                if raw > tol and nz > 0:
                    rep["err_over_noise"] = max(rep["err_over_noise"], en / nz)
    rep["ok"] = bool(rep["worst_ratio"] <= 1.0)
    return rep


def bf16_tensor(bits: np.ndarray, device):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device`."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
