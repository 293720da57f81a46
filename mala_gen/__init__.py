"""Seeded synthetic inputs for MALA (MassAlloc Attention).

This module only draws random tensors and rounds them to bf16.  It holds none of
the attention arithmetic: both the fp64 oracle and the HIP path consume exactly
the bf16 bit patterns produced here, the oracle after an exact upcast to fp64.

The pages ("MassAlloc Attention: Let Attention Allocate Its Own Compute", all
five pages) measure on activations of trained models, which are not available.
The recipes below are synthetic stand-ins with the structure the pages
describe as typical of long-context attention (page 2, "Core idea", and page 1,
second paragraph): mass concentrated on local keys, a few sink tokens and a few
retrieval targets.  Diffuse heads (i.i.d. normal Q and K) are the opposite
extreme, where every tile is retained.

Recipe "local/sink/retrieval" for one KV head of width d and length L:
  * u is a random unit vector,
  * K, V ~ N(0, I); the first four keys are sinks: K[0:4] += 3 u,
  * for each query row i of each q head sharing the KV head: with probability
    p the row targets a uniformly random earlier key t in [0, i-1] (t = 0 for
    i = 0); otherwise t = max(i - r, 0) with r uniform in 0..31,
  * Q[i] = 2.5 sqrt(d) K[t]/|K[t]| + 1.5 u + N(0, 0.5^2 I),
  * dO ~ N(0, I).
Recipe "diffuse": Q, K, V, dO ~ N(0, I).
Decode recipe (one new token against a cache of N keys): cache K, V as in the
local/sink/retrieval recipe; the query of each q head is
  q = 2.5 sqrt(d) sum_{t in T} K[t]/|K[t]| + 1.5 u + N(0, 0.5^2 I)
with T = {one t uniform in [N-256, N)} plus four t uniform in [4, N-256).

Every draw comes from numpy's PCG64 seeded with SeedSequence([tag, b, kv_head,
0x4D414C41]); the draw order per KV head is fixed (u, K, V, then per q head the
retrieval coin, the retrieval target, the local offset, the noise, then dO).
"""
from __future__ import annotations

import numpy as np

SEED_SALT = 0x4D414C41


# --------------------------------------------------------------------------
# bf16 rounding (round to nearest even), carried as uint16 bit patterns.
# --------------------------------------------------------------------------
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> bf16 bit pattern (uint16), round-to-nearest-even.

    The value is first rounded to float32 (RNE) and then to bf16 (RNE); inputs
    are finite.  Both consumers see the same bits, so the double rounding only
    defines which bf16 value the input is.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(tag: int, b: int, kvh: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([tag, b, kvh, SEED_SALT])))


# --------------------------------------------------------------------------
# Training / prefill inputs: Q, K, V, dO in [B, L, H, d] (d contiguous).
# --------------------------------------------------------------------------
def _local_retrieval_head(rng, L, G, d, p):
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    K = rng.standard_normal((L, d))
    K[: min(4, L)] += 3.0 * u
    V = rng.standard_normal((L, d))
    Kn = K / np.linalg.norm(K, axis=1, keepdims=True)
    i = np.arange(L)
    Q = np.empty((L, G, d))
    for g in range(G):
        retr = rng.random(L) < p
        t_retr = np.floor(rng.random(L) * i).astype(np.int64)  # uniform in [0, i-1]; 0 when i == 0
        r = rng.integers(0, 32, size=L)
        t_loc = np.maximum(i - r, 0)
        t = np.where(retr, t_retr, t_loc)
        Q[:, g, :] = 2.5 * np.sqrt(d) * Kn[t] + 1.5 * u + 0.5 * rng.standard_normal((L, d))
    dO = rng.standard_normal((L, G, d))
    return Q, K, V, dO


def _diffuse_head(rng, L, G, d):
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    Q = rng.standard_normal((L, G, d))
    dO = rng.standard_normal((L, G, d))
    return Q, K, V, dO


def attn_inputs(tag: int, B: int, L: int, Hq: int, Hkv: int, d: int, p: float,
                diffuse_kv_heads=(), with_dout: bool = True) -> dict:
    """bf16 bit patterns q, k, v, dout with layout [B, L, H, d].

    `tag` seeds the stream (the workload's number); `diffuse_kv_heads` lists KV
    heads (and with them their q heads) drawn from the diffuse recipe.
    """
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    q = np.empty((B, L, Hq, d), np.uint16)
    k = np.empty((B, L, Hkv, d), np.uint16)
    v = np.empty((B, L, Hkv, d), np.uint16)
    do = np.empty((B, L, Hq, d), np.uint16) if with_dout else None
    diffuse = set(diffuse_kv_heads)
    for b in range(B):
        for kh in range(Hkv):
            rng = _rng(tag, b, kh)
            if kh in diffuse:
                Q, K, V, dO = _diffuse_head(rng, L, G, d)
            else:
                Q, K, V, dO = _local_retrieval_head(rng, L, G, d, p)
            q[b, :, kh * G:(kh + 1) * G, :] = round_to_bf16_bits(Q)
            k[b, :, kh, :] = round_to_bf16_bits(K)
            v[b, :, kh, :] = round_to_bf16_bits(V)
            if with_dout:
                do[b, :, kh * G:(kh + 1) * G, :] = round_to_bf16_bits(dO)
    return {"q": q, "k": k, "v": v, "dout": do,
            "B": B, "L": L, "Hq": Hq, "Hkv": Hkv, "d": d}


def varlen_inputs(tag: int, lens_q, lens_k, Hq: int, Hkv: int, d: int, p: float,
                  diffuse_kv_heads=()) -> dict:
    """Packed bf16 bit patterns for a batch of sequences whose Lq queries are
    the last Lq positions of their Lk keys: q [sum Lq, Hq, d], k/v
    [sum Lk, Hkv, d], cu_q/cu_k int32 [B+1].  Sequence s of length Lk is drawn
    exactly as attn_inputs draws batch entry s of a length-Lk sequence, so a
    chunk's rows are the last rows of that full sequence."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    lens_q, lens_k = [int(x) for x in lens_q], [int(x) for x in lens_k]
    if len(lens_q) != len(lens_k) or any(lq < 0 or lk < lq for lq, lk in zip(lens_q, lens_k)):
        raise ValueError("need 0 <= Lq <= Lk per sequence")
    G = Hq // Hkv
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = np.zeros((int(cu_q[-1]), Hq, d), np.uint16)
    k = np.zeros((int(cu_k[-1]), Hkv, d), np.uint16)
    v = np.zeros((int(cu_k[-1]), Hkv, d), np.uint16)
    do = np.zeros((int(cu_q[-1]), Hq, d), np.uint16)
    diffuse = set(diffuse_kv_heads)
    for s, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        if lk == 0:
            continue
        for kh in range(Hkv):
            rng = _rng(tag, s, kh)
            if kh in diffuse:
                Q, K, V, dO = _diffuse_head(rng, lk, G, d)
            else:
                Q, K, V, dO = _local_retrieval_head(rng, lk, G, d, p)
            q[cu_q[s]:cu_q[s + 1], kh * G:(kh + 1) * G, :] = round_to_bf16_bits(Q[lk - lq:])
            k[cu_k[s]:cu_k[s + 1], kh, :] = round_to_bf16_bits(K)
            v[cu_k[s]:cu_k[s + 1], kh, :] = round_to_bf16_bits(V)
            do[cu_q[s]:cu_q[s + 1], kh * G:(kh + 1) * G, :] = round_to_bf16_bits(dO[lk - lq:])
    return {"q": q, "k": k, "v": v, "dout": do, "cu_q": cu_q, "cu_k": cu_k, "Hq": Hq, "Hkv": Hkv, "d": d}


def decode_inputs(tag: int, B: int, N: int, Hq: int, Hkv: int, d: int) -> dict:
    """bf16 bit patterns: q [B, Hq, d], kcache/vcache [B, N, Hkv, d]."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    q = np.empty((B, Hq, d), np.uint16)
    k = np.empty((B, N, Hkv, d), np.uint16)
    v = np.empty((B, N, Hkv, d), np.uint16)
    for b in range(B):
        for kh in range(Hkv):
            rng = _rng(tag, b, kh)
            u = rng.standard_normal(d)
            u /= np.linalg.norm(u)
            K = rng.standard_normal((N, d))
            K[: min(4, N)] += 3.0 * u
            V = rng.standard_normal((N, d))
            for g in range(G):
                lo = max(N - 256, 0)
                t_recent = rng.integers(lo, N)
                far_hi = max(N - 256, 5)
                t_far = rng.integers(4, far_hi, size=4) if N > 8 else rng.integers(0, N, size=4)
                T = np.concatenate([[t_recent], t_far])
                Kt = K[T]
                qv = 2.5 * np.sqrt(d) * (Kt / np.linalg.norm(Kt, axis=1, keepdims=True)).sum(0)
                qv = qv + 1.5 * u + 0.5 * rng.standard_normal(d)
                q[b, kh * G + g] = round_to_bf16_bits(qv)
            k[b, :, kh, :] = round_to_bf16_bits(K)
            v[b, :, kh, :] = round_to_bf16_bits(V)
    return {"q": q, "k": k, "v": v, "B": B, "N": N, "Hq": Hq, "Hkv": Hkv, "d": d}


# --------------------------------------------------------------------------
# The named workloads (shapes, tiles and tolerances of each).
# --------------------------------------------------------------------------
WORKLOADS = {
    "tiny_512": dict(tag=0, B=1, L=512, Hq=2, Hkv=2, d=64, p=0.1, diffuse=(), Bq=64, Bk=64, taus=(0.0, 1.0)),
    "gqa_8k": dict(tag=1, B=1, L=8192, Hq=16, Hkv=4, d=128, p=0.1, diffuse=(2, 3), Bq=128, Bk=64, taus=(1.0,)),
    "sweep": dict(tag=2, B=1, Hq=16, Hkv=4, d=128, p=0.1, diffuse=(2, 3), Bq=128, Bk=64,
                  Ls=(1024, 2048, 4096, 8192, 16384, 32768), taus=(0.0, 0.25, 1.0, 4.0)),
    "train_128k": dict(tag=3, B=1, L=131072, Hq=5, Hkv=1, d=128, p=0.02, diffuse=(), Bq=128, Bk=64, taus=(1.0, 0.0)),
    "decode_128k": dict(tag=4, B=8, N=131072, Hq=5, Hkv=1, d=128, Bk_dec=64, taus=(1.0, 0.0)),
    # the last 16K queries of the 128K training sequence, prefilled onto the
    # cache of the 112K keys before them (same seeds as train_128k)
    "prefill_128k": dict(tag=3, lens_q=(16384,), lens_k=(131072,), Hq=5, Hkv=1, d=128, p=0.02, diffuse=(),
                         Bq=128, Bk=64, taus=(1.0, 0.0)),
    # a ragged batch: fresh prompts (Lq = Lk), chunks onto caches, single tokens
    "varlen_mix": dict(tag=5, lens_q=(1000, 333, 1, 2048, 0, 700), lens_k=(1000, 2900, 5000, 5000, 77, 700),
                       Hq=8, Hkv=2, d=128, p=0.1, diffuse=(1,), Bq=128, Bk=64, taus=(0.0, 0.25, 1.0, 4.0)),
}


def workload_inputs(name: str, L: int | None = None, with_dout: bool = True) -> dict:
    w = WORKLOADS[name]
    if "lens_q" in w:
        return varlen_inputs(w["tag"], w["lens_q"], w["lens_k"], w["Hq"], w["Hkv"], w["d"], w["p"], w["diffuse"])
    if name == "decode_128k":
        return decode_inputs(w["tag"], w["B"], w["N"] if L is None else L, w["Hq"], w["Hkv"], w["d"])
    LL = w.get("L") if L is None else L
    return attn_inputs(w["tag"], w["B"], LL, w["Hq"], w["Hkv"], w["d"], w["p"], w["diffuse"], with_dout)
