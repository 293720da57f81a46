"""Comparison helpers for GPU-vs-oracle parity.

Decision parity: a GPU decision that differs from the oracle's is *exempt* when
the oracle's log-margin lies within ln(1 + 1e-3) of zero (the ratio is within
1e-3 relative of the threshold); once a block has an exempt mismatch, later
mismatches in the same block (in visit order) are *cascade* mismatches, since
the two runs no longer share the retained state.  Any other mismatch is
non-exempt and fails the test.
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


def rel_l2(x: np.ndarray, y: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    n = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / n) if n > 0 else float(np.linalg.norm(x - y))


def rel_l2_per_head(x, y, head_axis: int = 2, floor_frac: float = 0.0):
    """Max over (b, h) slices of the relative L2 error, and the global value.

    With floor_frac > 0 each slice's error is divided by
    max(|y_slice|, floor_frac * max_slices |y_slice|): a slice whose exact value
    is vanishingly small next to the others (a gradient that cancels to ~1e-7 of
    its neighbours, below what fp32 arithmetic resolves) is measured against
    that floor instead of its own norm."""
    x = np.moveaxis(np.asarray(x, np.float64), head_axis, 1)
    y = np.moveaxis(np.asarray(y, np.float64), head_axis, 1)
    norms = np.array([[np.linalg.norm(y[b, h]) for h in range(y.shape[1])] for b in range(y.shape[0])])
    floor = floor_frac * norms.max() if norms.size else 0.0
    worst = 0.0
    for b in range(x.shape[0]):
        for h in range(x.shape[1]):
            den = max(norms[b, h], floor)
            err = np.linalg.norm(x[b, h] - y[b, h])
            worst = max(worst, err / den if den > 0 else err)
    return worst, rel_l2(x, y)


FP32_CANCEL = 2.0 ** -11


def grad_floors(name, q, k, v, dout, rowmask, scale):
    """Per-slice noise floor of an fp32 evaluation of the attention gradient.

    dS = P (dP - D) subtracts two dot products of magnitude |dO||v|; in fp32
    each carries ~1e-6 of that magnitude, so rows whose exact dS cancels
    (one-hot attention) have dq, dk far below what fp32 resolves.  The floor
    of a dq slice (b, h) is FP32_CANCEL * scale * |dO rows| * max|v| * max|k|;
    of a dk slice (b, kh) the same with the rows of every q head of the group
    and max|q|.  dv needs none (it has no cancellation).
    q, dout [B, L, Hq, d]; k, v [B, L, Hkv, d]; rowmask [B, L, Hq] rows compared.
    Returns [B, H] floors."""
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    Gq = Hq // Hkv
    vmax = np.linalg.norm(v, axis=-1).max(axis=1)          # [B, Hkv]
    kmax = np.linalg.norm(k, axis=-1).max(axis=1)
    qmax = np.linalg.norm(q, axis=-1).max(axis=1)           # [B, Hq]
    dn = np.sqrt((np.where(rowmask[..., None], dout, 0.0) ** 2).sum(axis=(1, 3)))   # [B, Hq]
    if name == "dq":
        kh = np.arange(Hq) // Gq
        return FP32_CANCEL * scale * dn * vmax[:, kh] * kmax[:, kh]
    if name == "dk":
        dng = np.sqrt((dn ** 2).reshape(B, Hkv, Gq).sum(-1))
        qg = qmax.reshape(B, Hkv, Gq).max(-1)
        return FP32_CANCEL * scale * dng * vmax * qg
    return np.zeros((B, Hkv))


def rel_l2_floored(x, y, floors, head_axis: int = 2):
    """Max over (b, h) slices of |x - y| / max(|y|, floor[b, h]), and the global
    relative error."""
    x = np.moveaxis(np.asarray(x, np.float64), head_axis, 1)
    y = np.moveaxis(np.asarray(y, np.float64), head_axis, 1)
    worst = 0.0
    for b in range(x.shape[0]):
        for h in range(x.shape[1]):
            den = max(np.linalg.norm(y[b, h]), floors[b, h])
            err = np.linalg.norm(x[b, h] - y[b, h])
            worst = max(worst, err / den if den > 0 else err)
    return worst, rel_l2(x, y)


def bf16_tensor(bits: np.ndarray, device):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device`."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
