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


def rel_l2_per_head(x, y, head_axis: int = 2):
    """Max over (b, h) slices of the relative L2 error, and the global value."""
    x = np.moveaxis(np.asarray(x, np.float64), head_axis, 1)
    y = np.moveaxis(np.asarray(y, np.float64), head_axis, 1)
    worst = 0.0
    for b in range(x.shape[0]):
        for h in range(x.shape[1]):
            worst = max(worst, rel_l2(x[b, h], y[b, h]))
    return worst, rel_l2(x, y)


def bf16_tensor(bits: np.ndarray, device):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on `device`."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
