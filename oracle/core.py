"""ctypes binding of the fp64 C oracle (mala_oracle.c) -- test infrastructure only.

Every array is float64 / int32 / uint8 numpy, C-contiguous.  Layouts follow
the C file: q, o, dout, dq [B, L, Hq, d]; k, v, dk, dv [B, L, Hkv, d];
lse [B, Hq, L]; per-tile keep/margin [B, Hq, nQB, nKT]; decode q/o [B, Hq, d],
caches [B, N, Hkv, d], keep/margin [B, Hkv, nT].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mala_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libmala_oracle.so")
KEEP_UNVISITED = 255

_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain IEEE fp64, OpenMP)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # MALA_ORACLE_LIB names another build of mala_oracle.c to load instead
    # (the mutation tests point it at deliberately broken copies)
    path = os.environ.get("MALA_ORACLE_LIB")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build_oracle(force=True)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, f64 = ctypes.c_int, ctypes.c_double
    lib.mala_oracle_fwd.argtypes = [P, P, P, i32, i32, i32, i32, i32, f64, i32, i32, P, i32,
                                    P, P, P, P, P, P, i32]
    lib.mala_oracle_bwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, f64, i32, i32,
                                    P, i32, P, i32, P, P, P, P, P, P, P, i32]
    lib.mala_oracle_fwd_varlen.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f64, i32, i32, P, i32,
                                           P, P, P, P, P, P, i32]
    lib.mala_oracle_bwd_varlen.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, f64, i32, i32,
                                           P, i32, P, i32, P, P, P, P, P, P, P, i32]
    lib.mala_oracle_decode.argtypes = [P, P, P, i32, i32, i32, i32, i32, f64, i32, P,
                                       P, P, P, P, P, P, i32]
    lib.mala_oracle_fwd_forced.argtypes = [P, P, P, i32, i32, i32, i32, i32, f64, i32, i32, P, i32, P,
                                           P, P, P, P, P, P, i32]
    lib.mala_oracle_decode_forced.argtypes = [P, P, P, i32, i32, i32, i32, i32, f64, i32, P, P,
                                              P, P, P, P, P, P, i32]
    lib.mala_oracle_fwd_varlen_forced.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f64, i32, i32, P, i32, P,
                                                  P, P, P, P, P, P, i32]
    for f in (lib.mala_oracle_fwd, lib.mala_oracle_fwd_varlen, lib.mala_oracle_bwd, lib.mala_oracle_bwd_varlen,
              lib.mala_oracle_decode, lib.mala_oracle_fwd_forced, lib.mala_oracle_decode_forced,
              lib.mala_oracle_fwd_varlen_forced):
        f.restype = ctypes.c_int
    lib.mala_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def oracle_threads() -> int:
    return int(_load().mala_oracle_max_threads())


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def oracle_fwd(q, k, v, tau: float, Bq: int, Bk: int, blocks=None, forced=None, nthreads: int = 0):
    """Forward rule.  Returns dict(o, lse, keep, margin, kept_slots, omitted).

    `blocks`: optional list of flat block ids (b*Hq + h)*nQB + qb; only those
    query blocks are computed (rows of other blocks stay NaN / -1 / 255).
    `forced`: optional uint8 [B, Hq, nQB, nKT] teacher-forced replay (0 / 1 =
    the decision a tile's state update follows, 255 = the rule's); keep and
    margin are then the rule's own, given the forced trajectory, and o, lse
    and the statistics those of the forced run (mala_oracle_fwd_forced).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    o = np.full(q.shape, np.nan)
    lse = np.full((B, Hq, L), np.nan)
    keep = np.full((B, Hq, nQB, nKT), KEEP_UNVISITED, np.uint8)
    margin = np.full((B, Hq, nQB, nKT), np.nan)
    slots = np.full((B, Hq, L), -1, np.int32)
    omitted = np.full((B, Hq, L), np.nan)
    bl = None if blocks is None else np.ascontiguousarray(blocks, dtype=np.int32)
    if forced is None:
        rc = _load().mala_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), B, L, Hq, Hkv, d, float(tau), Bq, Bk,
                                     _ptr(bl), 0 if bl is None else len(bl),
                                     _ptr(o), _ptr(lse), _ptr(keep), _ptr(margin), _ptr(slots), _ptr(omitted),
                                     int(nthreads))
    else:
        fz = np.ascontiguousarray(forced, dtype=np.uint8)
        if fz.shape != (B, Hq, nQB, nKT):
            raise ValueError(f"forced must be [B, Hq, nQB, nKT] = {(B, Hq, nQB, nKT)}, got {fz.shape}")
        rc = _load().mala_oracle_fwd_forced(_ptr(q), _ptr(k), _ptr(v), B, L, Hq, Hkv, d, float(tau), Bq, Bk,
                                            _ptr(bl), 0 if bl is None else len(bl), _ptr(fz),
                                            _ptr(o), _ptr(lse), _ptr(keep), _ptr(margin), _ptr(slots),
                                            _ptr(omitted), int(nthreads))
    if rc:
        raise ValueError(f"oracle_fwd failed with code {rc}")
    return {"o": o, "lse": lse, "keep": keep, "margin": margin, "kept_slots": slots, "omitted": omitted}


def oracle_fwd_varlen(q, k, v, cu_q, cu_k, tau: float, Bq: int, Bk: int, blocks=None, forced=None,
                      nthreads: int = 0):
    """Variable-length forward (queries at the end of their keys, Lq <= Lk).

    q [total_q, Hq, d], k/v [total_k, Hkv, d]; cu_q/cu_k [B+1] cumulative
    lengths.  Returns dict(o, lse [Hq, total_q], keep/margin [B, Hq, nQB, nKT],
    kept_slots, omitted) with nQB, nKT from the longest sequence; `blocks` and
    `forced` (keep's layout) as in oracle_fwd with that nQB.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = np.ascontiguousarray(cu_q, dtype=np.int32)
    ck = np.ascontiguousarray(cu_k, dtype=np.int32)
    B = len(cq) - 1
    Tq, Hq, d = q.shape
    Hkv = k.shape[1]
    maxq = int(np.max(np.diff(cq))) if B > 0 else 0
    maxk = int(np.max(np.diff(ck))) if B > 0 else 0
    nQB, nKT = max(1, -(-maxq // Bq)), max(1, -(-maxk // Bk))
    o = np.full(q.shape, np.nan)
    lse = np.full((Hq, Tq), np.nan)
    keep = np.full((B, Hq, nQB, nKT), KEEP_UNVISITED, np.uint8)
    margin = np.full((B, Hq, nQB, nKT), np.nan)
    slots = np.full((Hq, Tq), -1, np.int32)
    omitted = np.full((Hq, Tq), np.nan)
    bl = None if blocks is None else np.ascontiguousarray(blocks, dtype=np.int32)
    if forced is None:
        rc = _load().mala_oracle_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cq), _ptr(ck), B, Hq, Hkv, d,
                                            float(tau), Bq, Bk, _ptr(bl), 0 if bl is None else len(bl),
                                            _ptr(o), _ptr(lse), _ptr(keep), _ptr(margin), _ptr(slots),
                                            _ptr(omitted), int(nthreads))
    else:
        fz = np.ascontiguousarray(forced, dtype=np.uint8)
        if fz.shape != keep.shape:
            raise ValueError(f"forced must be [B, Hq, nQB, nKT] = {keep.shape}, got {fz.shape}")
        rc = _load().mala_oracle_fwd_varlen_forced(_ptr(q), _ptr(k), _ptr(v), _ptr(cq), _ptr(ck), B, Hq, Hkv, d,
                                                   float(tau), Bq, Bk, _ptr(bl), 0 if bl is None else len(bl),
                                                   _ptr(fz), _ptr(o), _ptr(lse), _ptr(keep), _ptr(margin),
                                                   _ptr(slots), _ptr(omitted), int(nthreads))
    if rc:
        raise ValueError(f"oracle_fwd_varlen failed with code {rc}")
    return {"o": o, "lse": lse, "keep": keep, "margin": margin, "kept_slots": slots, "omitted": omitted}


def oracle_bwd(q, k, v, o, dout, lse, tau: float, Bq: int, Bk: int,
               qunits=None, kunits=None, do_dq=True, do_dkdv=True, cond: bool = False, nthreads: int = 0):
    """Backward rule.  Returns dict(dq, dk, dv, keep, margin), plus dq_cond and
    dk_cond (the first-order error scales of a binary32 evaluation of dP - D,
    described in mala_oracle.c) when `cond` is set.

    `qunits` (flat (b*Hq + h)*nQB + qb) restricts the dq pass, `kunits`
    (flat (b*Hkv + kh)*nKT + kt) the dk/dv pass; rows outside stay NaN.
    """
    q, k, v, o, dout, lse = map(_f64, (q, k, v, o, dout, lse))
    B, L, Hq, d = q.shape
    Hkv = k.shape[2]
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(k.shape, np.nan)
    dqc = np.full(q.shape, np.nan) if cond else None
    dkc = np.full(k.shape, np.nan) if cond else None
    keep = np.full((B, Hq, nQB, nKT), KEEP_UNVISITED, np.uint8)
    margin = np.full((B, Hq, nQB, nKT), np.nan)
    qa = None if qunits is None else np.ascontiguousarray(qunits, dtype=np.int32)
    ka = None if kunits is None else np.ascontiguousarray(kunits, dtype=np.int32)
    nq = (len(qa) if qa is not None else 0) if do_dq else -1
    nk = (len(ka) if ka is not None else 0) if do_dkdv else -1
    if not do_dq:
        qa = None
    if not do_dkdv:
        ka = None
    rc = _load().mala_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                 B, L, Hq, Hkv, d, float(tau), Bq, Bk,
                                 _ptr(qa), nq, _ptr(ka), nk,
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(keep), _ptr(margin),
                                 _ptr(dqc), _ptr(dkc), int(nthreads))
    if rc:
        raise ValueError(f"oracle_bwd failed with code {rc}")
    out = {"dq": dq, "dk": dk, "dv": dv, "keep": keep, "margin": margin}
    if cond:
        out["dq_cond"], out["dk_cond"] = dqc, dkc
    return out


def oracle_bwd_varlen(q, k, v, o, dout, lse, cu_q, cu_k, tau: float, Bq: int, Bk: int,
                      qunits=None, kunits=None, do_dq=True, do_dkdv=True, cond: bool = False, nthreads: int = 0):
    """Variable-length backward over the packed layout of oracle_fwd_varlen
    (lse [Hq, total_q]).  Returns dict(dq, dk, dv, keep, margin), plus
    dq_cond / dk_cond with `cond` as in oracle_bwd; unit ids as in oracle_bwd
    with nQB, nKT from the longest sequence."""
    q, k, v, o, dout, lse = map(_f64, (q, k, v, o, dout, lse))
    cq = np.ascontiguousarray(cu_q, dtype=np.int32)
    ck = np.ascontiguousarray(cu_k, dtype=np.int32)
    B = len(cq) - 1
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    maxq = int(np.max(np.diff(cq))) if B > 0 else 0
    maxk = int(np.max(np.diff(ck))) if B > 0 else 0
    nQB, nKT = max(1, -(-maxq // Bq)), max(1, -(-maxk // Bk))
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(k.shape, np.nan)
    dqc = np.full(q.shape, np.nan) if cond else None
    dkc = np.full(k.shape, np.nan) if cond else None
    keep = np.full((B, Hq, nQB, nKT), KEEP_UNVISITED, np.uint8)
    margin = np.full((B, Hq, nQB, nKT), np.nan)
    qa = None if qunits is None else np.ascontiguousarray(qunits, dtype=np.int32)
    ka = None if kunits is None else np.ascontiguousarray(kunits, dtype=np.int32)
    nq = (len(qa) if qa is not None else 0) if do_dq else -1
    nk = (len(ka) if ka is not None else 0) if do_dkdv else -1
    if not do_dq:
        qa = None
    if not do_dkdv:
        ka = None
    rc = _load().mala_oracle_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                        _ptr(cq), _ptr(ck), B, Hq, Hkv, d, float(tau), Bq, Bk,
                                        _ptr(qa), nq, _ptr(ka), nk,
                                        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(keep), _ptr(margin),
                                        _ptr(dqc), _ptr(dkc), int(nthreads))
    if rc:
        raise ValueError(f"oracle_bwd_varlen failed with code {rc}")
    out = {"dq": dq, "dk": dk, "dv": dv, "keep": keep, "margin": margin}
    if cond:
        out["dq_cond"], out["dk_cond"] = dqc, dkc
    return out


def oracle_decode(q, kc, vc, tau: float, Bkd: int, seqlens=None, forced=None, nthreads: int = 0):
    """Decode rule.  Returns dict(o, lse, keep, margin, kept_tiles, omitted).

    `seqlens`: optional [B] cache lengths (1 <= N_b <= N); sequence b then
    sees only its first N_b cache rows (tiles past them stay 255 / NaN).
    `forced`: optional uint8 [B, Hkv, nT] teacher-forced replay, as in
    oracle_fwd (mala_oracle_decode_forced)."""
    q, kc, vc = _f64(q), _f64(kc), _f64(vc)
    sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
    B, Hq, d = q.shape
    N, Hkv = kc.shape[1], kc.shape[2]
    nT = -(-N // Bkd)
    o = np.full(q.shape, np.nan)
    lse = np.full((B, Hq), np.nan)
    keep = np.full((B, Hkv, nT), KEEP_UNVISITED, np.uint8)
    margin = np.full((B, Hkv, nT), np.nan)
    kept = np.full((B, Hkv), -1, np.int32)
    omitted = np.full((B, Hq), np.nan)
    if forced is not None:
        fz = np.ascontiguousarray(forced, dtype=np.uint8)
        if fz.shape != (B, Hkv, nT):
            raise ValueError(f"forced must be [B, Hkv, nT] = {(B, Hkv, nT)}, got {fz.shape}")
        rc = _load().mala_oracle_decode_forced(_ptr(q), _ptr(kc), _ptr(vc), B, N, Hq, Hkv, d, float(tau), Bkd,
                                               _ptr(sl), _ptr(fz), _ptr(o), _ptr(lse), _ptr(keep), _ptr(margin),
                                               _ptr(kept), _ptr(omitted), int(nthreads))
        if rc:
            raise ValueError(f"oracle_decode failed with code {rc}")
        return {"o": o, "lse": lse, "keep": keep, "margin": margin, "kept_tiles": kept, "omitted": omitted}
    rc = _load().mala_oracle_decode(_ptr(q), _ptr(kc), _ptr(vc), B, N, Hq, Hkv, d, float(tau), Bkd, _ptr(sl),
                                    _ptr(o), _ptr(lse), _ptr(keep), _ptr(margin), _ptr(kept), _ptr(omitted),
                                    int(nthreads))
    if rc:
        raise ValueError(f"oracle_decode failed with code {rc}")
    return {"o": o, "lse": lse, "keep": keep, "margin": margin, "kept_tiles": kept, "omitted": omitted}
