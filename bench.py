"""Benchmark of the MALA hot path on one MI355X.

One step = one pass of the whole path on synthetic inputs resident in HBM:
  * training forward + backward at 128K tokens (B=1, Hq=5, Hkv=1, d=128 --
    one GPU's share of a 40q/8kv-head model split 8 ways by heads), tau = 1,
  * one decode step of 8 sequences against a 131072-token cache (Hq=5,
    Hkv=1, d=128), tau = 1.
`value` is the step's throughput in the method's own (algorithmic) FLOPs per
second: scores of every legal query-key pair (2d each, the skip decision
needs them) plus the post-score work of retained pairs (forward 2d for P.V;
backward 8d for dP, dV, dK and dQ; decode: scores of every cached key and
head, 2d P.V per retained key and head), divided by the measured step time.
It is what the GPU actually does per second and stays below the MFMA peak.
`effective_tflops` gives the dense-equivalent rates the metric name refers
to (the FLOPs dense causal attention would spend on the same outputs:
forward 4d per legal pair, backward 10d) -- skipped work is credited there,
so those rates can exceed the peak.  The same kernels at tau = 0 (the dense
path) are timed in the same run for the speedups, the dominant kernel's
roofline is measured live with HIP events on the launch stream, each
operator's device memory (outputs + workspace) and the allocator's peak
around the step are reported for tau = 1 and tau = 0, and the fp64 oracle is
timed on a bounded sample of the same workload on the host cores.

`--workload prefill_128k` instead times the variable-length forward on a
chunked prefill: the last 16384 queries of the 128K sequence against all of its
131072 keys (the cache of the 114688 keys before them plus the chunk itself),
and prints that measurement's own JSON line.

`--workload tau_sweep` measures fidelity against cost over the sweep workload
(Hq=16, Hkv=4, half the heads diffuse; L = 1K .. 32K): per (L, tau) the forward
time, kept tiles, retained key slots per query, the omitted probability mass
(kernel statistics mode) and the relative L2 distance of O from the tau = 0
output of the same kernel, per head.

`--workload matched_work` compares allocation policies at matched post-score
work (8K context, 16 q heads over 4 KV heads): MALA's own online decisions at
tau = 1 set the budget (its retained key slots), and three policies that pick
key tiles by their finalized reference mass (the exact softmax mass of the
tile) spend exactly that budget: the same slots per query everywhere
(static), a per-(head, query block) profile measured on separate calibration
inputs (head-position), and one ranking over the whole instance (per-instance
oracle).  Every policy keeps each block's newest (diagonal) tile.  Reported:
omitted probability mass and relative L2 error of O against dense attention.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-tau0]
                       [--workload step|prefill_128k|tau_sweep|matched_work]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MALA fwd/bwd ms + effective TFLOP/s at 128K (1 GPU share), decode ms vs τ=0"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--tau", type=float, default=1.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-tau0", action="store_true", help="skip the tau=0 comparison")
    ap.add_argument("--cpu-blocks", type=int, default=48, help="query blocks per head in the CPU sample")
    ap.add_argument("--workload", choices=("step", "prefill_128k", "tau_sweep", "matched_work"), default="step",
                    help="step: training forward+backward and decode (default); prefill_128k: chunked prefill; "
                         "tau_sweep: fidelity and cost against tau")
    ap.add_argument("--taus", type=str, default="0.01,0.05,0.25,1,4,16",
                    help="tau values of the tau_sweep workload (tau = 0 is always run as the reference)")
    ap.add_argument("--traffic-probe", nargs="?", const="fwd", default=None, choices=("fwd", "decode", "bwd"),
                    help="run two forward (or two decode, each after a 512 MB read flush; or one forward and "
                         "two backward) launches and a plain 1 GiB device copy, then exit (for PMC passes)")
    return ap.parse_args()


# The forward kernel's HBM traffic comes from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE) over `bench.py --traffic-probe`, calibrated against
# the plain copy kernel the probe runs; the summary records the figures and a
# hash of the kernel sources they were taken with.  A source change voids them.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mala_fwd_kernel_train_128k_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "adaptive_tile_skipping_amd", "csrc", f)
                  for f in ("mala_fwd.hip", "mala_device.h", "mala_internal.h", "mala_api.hip")]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """Bytes per forward launch from the committed PMC summary, or None when
    the summary is missing or was taken with other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        line = line.strip().strip("`")
        if ":" in line:
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measure_sustained(mala, dev, kcache, flush, reps: int = 5):
    """What the part sustains, from the library's two measurement probes
    (include/mala.h: mala_probe_mfma, mala_probe_read): back-to-back bf16
    MFMAs on register operands with no memory traffic, and a plain streaming
    read of a 1 GiB buffer (four times the last-level cache), and the same
    read of the decode's K cache alone after `flush()` (the bytes the decode's
    score pass must read, in one launch of their own size).  Median of `reps`
    timed launches after one untimed launch of each."""
    import numpy as np
    import torch
    fsink = torch.empty(mala.PROBE_SINK_WORDS, dtype=torch.float32, device=dev)
    isink = torch.empty(mala.PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    buf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        work = fn()
        e1.record()
        torch.cuda.synchronize()
        return work, e0.elapsed_time(e1)

    iters = 150000                        # ~20 ms per launch at ~1.9 PFLOP/s
    timed(lambda: mala.probe_mfma(iters, fsink))
    mfma = [w / (ms * 1e-3) / 1e12 for w, ms in (timed(lambda: mala.probe_mfma(iters, fsink)) for _ in range(reps))]
    timed(lambda: mala.probe_read(buf, isink))
    rd = [w / (ms * 1e-3) / 1e9 for w, ms in (timed(lambda: mala.probe_read(buf, isink)) for _ in range(reps))]
    del buf
    kus = []
    for _ in range(reps + 1):
        flush()
        kus.append(timed(lambda: mala.probe_read(kcache, isink))[1] * 1e3)
    return {"mfma_bf16_tflops": round(float(np.median(mfma)), 1), "hbm_read_gbs": round(float(np.median(rd)), 1),
            "read_kcache_us": round(float(np.median(kus[1:])), 2),
            "read_kcache_gbs": round(kcache.numel() * kcache.element_size() / (float(np.median(kus[1:])) * 1e-6)
                                     / 1e9, 1),
            "note": "library probes, same process: back-to-back 32x32x16 bf16 MFMAs on register operands (two "
                    "4-wave workgroups per CU, no memory traffic); a streaming read of 1 GiB (one 8-wave "
                    "workgroup per CU, 16-byte loads), and of the decode's 268 MB K cache alone after a 512 MB "
                    "flushing read; median of %d launches each" % reps}


def legal_pairs_block(L, Bq, qb):
    r0, r1 = qb * Bq, min(L, qb * Bq + Bq)
    return sum(i + 1 for i in range(r0, r1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kept_slots(keep, L, Bq, Bk, kept_value=1):
    """Legal query-key pairs inside the tiles marked kept in keep[B, H, nQB, nKT]."""
    import numpy as np
    nQB, nKT = keep.shape[-2], keep.shape[-1]
    rows = np.arange(L)
    j0 = np.arange(nKT)[None, :] * Bk
    per_row = np.clip(rows[:, None] - j0 + 1, 0, Bk)                   # [L, nKT] legal keys per row and tile
    pad = np.zeros((nQB * Bq, nKT), dtype=np.int64)
    pad[:L] = per_row
    tile_pairs = pad.reshape(nQB, Bq, nKT).sum(1)                       # [nQB, nKT]
    return float(((keep == kept_value) * tile_pairs).sum())


def cpu_baseline(args, inp, dinp, W, WD, tau):
    """The fp64 oracle timed on the host cores on a bounded sample of the
    benchmarked step, credited with the same algorithmic FLOPs as `value`.
    Legs: forward and backward dQ pass on evenly spaced query blocks of the
    128K sequence; forward and backward dK/dV pass on its first 16384 rows (a
    causal prefix is a problem of its own: its rows see no later key and
    their thresholds tau / (i + 1) do not change); the decode step on all
    eight sequences."""
    import numpy as np

    import mala_gen as G
    from oracle import oracle_bwd, oracle_decode, oracle_fwd, oracle_threads
    B, L, Hq, Hkv, d, Bq, Bk = W["B"], W["L"], W["Hq"], W["Hkv"], W["d"], W["Bq"], W["Bk"]
    nQB = -(-L // Bq)
    f64 = {x: G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v", "dout")}
    legs = {}

    # forward + dQ pass on sampled query blocks of the full sequence
    nb = max(1, args.cpu_blocks)
    qbs = [int((j + 0.5) * nQB / nb) for j in range(nb)]
    blocks = [h * nQB + qb for h in range(Hq) for qb in qbs]
    pairs_s = sum(legal_pairs_block(L, Bq, qb) for qb in qbs) * Hq
    t0 = time.perf_counter()
    rf = oracle_fwd(f64["q"], f64["k"], f64["v"], tau, Bq, Bk, blocks=blocks)
    t1 = time.perf_counter()
    rb = oracle_bwd(f64["q"], f64["k"], f64["v"], rf["o"], f64["dout"], rf["lse"], tau, Bq, Bk,
                    qunits=blocks, do_dkdv=False)
    t2 = time.perf_counter()
    legs["fwd_blocks"] = (2.0 * d * (pairs_s + kept_slots(rf["keep"], L, Bq, Bk)), t1 - t0)
    # each backward pass decides its tiles (scores of every legal pair) and
    # recomputes dP for kept ones: dQ pass S, dP, dQ; dK/dV pass S, dP, dV, dK
    legs["bwd_dq_blocks"] = (2.0 * d * pairs_s + 4.0 * d * kept_slots(rb["keep"], L, Bq, Bk), t2 - t1)

    # forward + dK/dV pass on the causal prefix
    Lp = min(L, 16384)
    pre = {x: np.ascontiguousarray(a[:, :Lp]) for x, a in f64.items()}
    pairs_p = B * Hq * Lp * (Lp + 1) // 2
    nKTp = -(-Lp // Bk)
    t0 = time.perf_counter()
    rp = oracle_fwd(pre["q"], pre["k"], pre["v"], tau, Bq, Bk)
    t1 = time.perf_counter()
    rpb = oracle_bwd(pre["q"], pre["k"], pre["v"], rp["o"], pre["dout"], rp["lse"], tau, Bq, Bk,
                     kunits=list(range(B * Hkv * nKTp)), do_dq=False)
    t2 = time.perf_counter()
    legs["fwd_prefix"] = (2.0 * d * (pairs_p + kept_slots(rp["keep"], Lp, Bq, Bk)), t1 - t0)
    legs["bwd_dkdv_prefix"] = (2.0 * d * pairs_p + 6.0 * d * kept_slots(rpb["keep"], Lp, Bq, Bk), t2 - t1)

    # decode: every sequence of the step
    dq64 = {x: G.bf16_bits_to_f64(dinp[x]) for x in ("q", "k", "v")}
    DB, DN, DHq, DHkv, Dd = WD["B"], WD["N"], WD["Hq"], WD["Hkv"], WD["d"]
    t0 = time.perf_counter()
    rd = oracle_decode(dq64["q"], dq64["k"], dq64["v"], tau, 64)
    t1 = time.perf_counter()
    kept_keys = float(np.minimum(rd["kept_tiles"].astype(np.int64) * 64, DN).sum())
    legs["decode"] = (2.0 * Dd * DN * DHq * DB + 2.0 * Dd * kept_keys * (DHq // DHkv), t1 - t0)

    flops = sum(fl for fl, _ in legs.values())
    secs = sum(sec for _, sec in legs.values())
    return {
        "value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": oracle_threads(),
        "cpu_model": cpu_model(), "kind": "oracle",
        "sample": f"fp64 oracle, tau={tau}: forward + backward dQ pass on {len(blocks)} query blocks of "
                  f"train_128k ({nb} evenly spaced blocks x {Hq} heads); forward + backward dK/dV pass on the "
                  f"first {Lp} rows; the decode_128k step (all {DB} sequences); credited with algorithmic FLOPs "
                  f"as the GPU value, each backward pass with its own decisions and dP; {secs:.1f} s",
        "legs": {n: {"tflop": round(fl / 1e12, 4), "seconds": round(sec, 2),
                     "tflops": round(fl / sec / 1e12, 6)} for n, (fl, sec) in legs.items()},
        "seconds": round(secs, 2)}



def main_prefill(args):
    """Chunked prefill through mala_fwd_varlen (see the module docstring)."""
    import numpy as np
    import torch

    import adaptive_tile_skipping_amd as mala
    import mala_gen as G

    dev = torch.device("cuda:0")
    torch.cuda.init()
    tau = args.tau
    W = G.WORKLOADS["prefill_128k"]
    Hq, Hkv, d, Bq, Bk = W["Hq"], W["Hkv"], W["d"], W["Bq"], W["Bk"]
    t_gen = time.time()
    inp = G.workload_inputs("prefill_128k")
    cu_q, cu_k = inp["cu_q"], inp["cu_k"]
    Lq, Lk = int(cu_q[-1]), int(cu_k[-1])
    off = Lk - Lq

    def tens(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = (tens(inp[x]) for x in ("q", "k", "v"))
    cq, ck = torch.from_numpy(cu_q).to(dev), torch.from_numpy(cu_k).to(dev)
    t_gen = time.time() - t_gen
    o = torch.empty_like(q)
    lse = torch.empty((Hq, Lq), dtype=torch.float32, device=dev)
    ws = mala.fwd_varlen_workspace(1, Lk, Hkv, d, Bq, Bk, dev)
    stream = torch.cuda.current_stream(dev)

    def run(t):
        mala.mala_fwd_varlen(q, k, v, cq, ck, Lq, Lk, t, Bq, Bk, o=o, lse=lse, ws=ws)

    def timed(t, steps, warmup):
        for _ in range(warmup):
            run(t)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for e0, e1 in ev:
            e0.record(stream); run(t); e1.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps * 1e3
        return wall, float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))

    wall, ms = timed(tau, max(args.steps, 5), args.warmup)
    print(f"# prefill tau={tau}: {ms:.3f} ms per call (wall {wall:.3f})", file=sys.stderr, flush=True)
    ms0 = None
    if not args.no_tau0:
        _, ms0 = timed(0.0, max(3, min(args.steps, 5)), 1)
        print(f"# prefill tau=0: {ms0:.3f} ms", file=sys.stderr, flush=True)

    st = mala.make_varlen_stats(1, Hq, Lq, Lq, Lk, Bq, Bk, dev)
    mala.mala_fwd_varlen(q, k, v, cq, ck, Lq, Lk, tau, Bq, Bk, o=o, lse=lse, stats=st, ws=ws)
    torch.cuda.synchronize()
    nQB = -(-Lq // Bq)
    n_visit = Hq * sum((off + min(Lq, qb * Bq + Bq) - 1) // Bk + 1 for qb in range(nQB))
    kf = int(st["kept_tiles"].sum().item())
    slots = float(st["kept_slots"].double().sum().item())
    pairs = Hq * (Lq * off + Lq * (Lq + 1) // 2)
    alg = 2.0 * d * pairs + 2.0 * d * slots
    achieved = alg / (ms * 1e-3) / 1e12
    out = {
        "metric": "MALA chunked prefill (16K queries onto a 128K-key sequence, 1 GPU share): effective TFLOP/s",
        "value": round(4.0 * d * pairs / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": max(args.steps, 5), "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"prefill_128k (B=1 Lq={Lq} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} Bq={Bq} Bk={Bk})",
                   "tau": tau},
        "wall_ms_per_call": round(wall, 4),
        "kept_tile_frac": round(kf / n_visit, 4),
        "slots_per_query": round(slots / (Hq * Lq), 1),
        "roofline": {"kernel": "mala_fwd_kernel (varlen launch, with its V copy)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_tflop_per_launch": round(alg / 1e12, 3), "launch_ms": round(ms, 4)},
        "gen_s": round(t_gen, 1),
    }
    if ms0 is not None:
        out["tau0_ms"] = round(ms0, 4)
        out["speedup_vs_tau0"] = round(ms0 / ms, 3)
    if not args.no_cpu:
        from oracle import oracle_fwd_varlen, oracle_threads
        f64 = {x: G.bf16_bits_to_f64(inp[x]) for x in ("q", "k", "v")}
        nb = max(1, args.cpu_blocks // 2)
        qbs = [int((j + 0.5) * nQB / nb) for j in range(nb)]
        blocks = [h * nQB + qb for h in range(Hq) for qb in qbs]
        pairs_s = Hq * sum(sum(off + i + 1 for i in range(qb * Bq, min(Lq, qb * Bq + Bq))) for qb in qbs)
        t0 = time.perf_counter()
        oracle_fwd_varlen(f64["q"], f64["k"], f64["v"], cu_q, cu_k, tau, Bq, Bk, blocks=blocks)
        tcpu = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": round(4.0 * d * pairs_s / tcpu / 1e12, 6), "unit": "TFLOP/s", "cores": oracle_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle varlen forward on {len(blocks)} query blocks of prefill_128k ({nb} evenly "
                      f"spaced blocks x {Hq} heads, tau={tau}); credited 4d FLOPs per legal pair; {tcpu:.1f} s",
            "seconds": round(tcpu, 2)}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# Matched-work allocation (summary/review: the matched-work control of the
# paper's Table 1 -- equal total post-score work, only its distribution over
# decisions differs).  Everything here is plain torch on per-tile arrays
# [H, nQB, nKT]; `legal` tiles are those a block visits.
# ---------------------------------------------------------------------------
def dense_tile_stats(q, k, v, Bq, Bk):
    """Exact softmax attention of one sequence, reduced to tiles.

    q [L, Hq, d], k/v [L, Hkv, d] (float tensors, any device).  Returns
    P-mass per tile mass[H, nQB, nKT], legal key slots per tile cost[H, nQB,
    nKT] (int64), the dense output o [L, Hq, d] and a function giving, for a
    tile keep mask, (omitted mass per row [Hq, L], renormalised output)."""
    import torch
    L, Hq, d = q.shape
    G = Hq // k.shape[1]
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    dev = q.device
    i = torch.arange(L, device=dev)
    causal = i[None, :] <= i[:, None]
    rows_pad, keys_pad = nQB * Bq, nKT * Bk
    cost1 = torch.zeros(rows_pad, keys_pad, dtype=torch.int64, device=dev)
    cost1[:L, :L] = causal.long()
    cost = cost1.view(nQB, Bq, nKT, Bk).sum(dim=(1, 3))
    probs = []
    mass = torch.zeros(Hq, nQB, nKT, dtype=torch.float64, device=dev)
    o = torch.empty(L, Hq, d, dtype=torch.float64, device=dev)
    for h in range(Hq):
        s = (q[:, h].double() @ k[:, h // G].double().T) / d ** 0.5
        s = s.masked_fill(~causal, float("-inf"))
        pr = torch.softmax(s, dim=-1)
        probs.append(pr)
        pp = torch.zeros(rows_pad, keys_pad, dtype=torch.float64, device=dev)
        pp[:L, :L] = pr
        mass[h] = pp.view(nQB, Bq, nKT, Bk).sum(dim=(1, 3))
        o[:, h] = pr @ v[:, h // G].double()

    def evaluate(keep):
        om = torch.empty(Hq, L, dtype=torch.float64, device=dev)
        out = torch.empty_like(o)
        for h in range(Hq):
            m = keep[h].repeat_interleave(Bq, 0).repeat_interleave(Bk, 1)[:L, :L]
            pk = torch.where(m, probs[h], torch.zeros((), dtype=torch.float64, device=dev))
            om[h] = torch.where(m, torch.zeros((), dtype=torch.float64, device=dev), probs[h]).sum(-1)
            out[:, h] = (pk @ v[:, h // G].double()) / pk.sum(-1, keepdim=True)
        return om, out

    return mass, cost.expand(Hq, nQB, nKT).contiguous(), o, evaluate


def diagonal_tiles(cost, Bq, Bk, L):
    """Tiles holding some row's own key, i.e. each row's first legal tile in
    visit order -- the tiles MALA always keeps and every policy keeps."""
    import torch
    H, nQB, nKT = cost.shape
    qb = torch.arange(nQB, device=cost.device)[:, None]
    kt = torch.arange(nKT, device=cost.device)[None, :]
    r0, r1 = qb * Bq, torch.clamp((qb + 1) * Bq, max=L)
    diag = (kt * Bk <= r1 - 1) & ((kt + 1) * Bk - 1 >= r0)
    return diag.expand(H, nQB, nKT) & (cost > 0)


def alloc_within_blocks(mass, cost, budget, forced):
    """Per block, the forced tiles plus the tiles of largest mass while the
    block's slots stay within budget[H, nQB]."""
    import torch
    rest = budget - (cost * forced).sum(-1)
    m = torch.where((cost > 0) & ~forced, mass, torch.full_like(mass, -1.0))
    order = torch.argsort(m, dim=-1, descending=True)
    c = torch.gather(torch.where((cost > 0) & ~forced, cost, torch.zeros_like(cost)), -1, order)
    take = (torch.cumsum(c, -1) <= rest[..., None]) & (torch.gather(m, -1, order) >= 0)
    keep = torch.zeros_like(forced)
    keep.scatter_(-1, order, take)
    return keep | forced


def alloc_global(mass, cost, total, forced):
    """Per-instance oracle: the forced tiles, then one ranking of every other
    legal tile by mass while the instance's slots stay within total."""
    import torch
    rest = total - int((cost * forced).sum())
    cand = (cost > 0) & ~forced
    m = torch.where(cand, mass, torch.full_like(mass, -1.0)).flatten()
    order = torch.argsort(m, descending=True)
    c = torch.where(cand, cost, torch.zeros_like(cost)).flatten()[order]
    take = (torch.cumsum(c, 0) <= rest) & (m[order] >= 0)
    keep = torch.zeros_like(m, dtype=torch.bool)
    keep[order] = take
    return keep.view(mass.shape) | forced


def static_budget(cost, total, Bq, L):
    """The same slots per query for every block (water-filled: blocks that
    cannot use their share give it to the others), summing to total."""
    import torch
    nQB = cost.shape[1]
    rows = torch.tensor([min(Bq, L - qb * Bq) for qb in range(nQB)], dtype=torch.float64, device=cost.device)
    cap = cost.sum(-1).double()                               # [H, nQB] legal slots
    lo, hi = 0.0, float(L)
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if float(torch.minimum(mid * rows, cap).sum()) < total:
            lo = mid
        else:
            hi = mid
    return torch.minimum(hi * rows, cap).floor().long()


def profile_budget(profile, cost, total):
    """A [H, nQB] slot profile scaled to the instance's total, capped at each
    block's legal slots."""
    import torch
    cap = cost.sum(-1)
    prof = profile / profile.sum()
    lo, hi = 0.0, 4.0 * total
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if float(torch.minimum(prof * mid, cap.double()).sum()) < total:
            lo = mid
        else:
            hi = mid
    return torch.minimum(prof * hi, cap.double()).floor().long()


def main_matched_work(args):
    """Matched-work allocation study (module docstring)."""
    import numpy as np
    import torch

    import adaptive_tile_skipping_amd as mala
    import mala_gen as G

    dev = torch.device("cuda:0")
    torch.cuda.init()
    L, Hq, Hkv, d, Bq, Bk, p = 8192, 16, 4, 128, 128, 64, 0.02
    tau = args.tau
    calib, evals = [700, 701, 702, 703], [710, 711, 712, 713]

    def instance(tag):
        inp = G.attn_inputs(tag, 1, L, Hq, Hkv, d, p, with_dout=False)
        t = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa
        q, k, v = (t(inp[x]) for x in ("q", "k", "v"))
        st = mala.make_stats(1, Hq, L, Bq, Bk, dev)
        mala.mala_fwd(q, k, v, tau, Bq, Bk, stats=st)
        torch.cuda.synchronize()
        nKT = -(-L // Bk)
        bits = st["decision_bits"][0].long() & 0xFFFFFFFF                     # [Hq, nQB, words]
        kt = torch.arange(nKT, device=dev)
        mala_keep = ((bits[..., kt // 32] >> (kt % 32)) & 1).bool()
        mass, cost, o, evaluate = dense_tile_stats(q[0].float(), k[0].float(), v[0].float(), Bq, Bk)
        return mala_keep & (cost > 0), mass, cost, o, evaluate

    # two work budgets: MALA's own retained slots at tau, and a fixed 1024
    # slots per query (the reference policies only)
    FIXED = 1024 * Hq * L
    insts = {}

    def budgets(mk, cost):
        return {"mala": int((cost * mk).sum()), "fixed_1024": FIXED}

    # calibration: the per-instance oracle's mean allocation per (head, block), per budget
    prof = {}
    for tag in calib:
        mk, mass, cost, _, _ = instance(tag)
        fz = diagonal_tiles(cost, Bq, Bk, L)
        for bname, total in budgets(mk, cost).items():
            a = (cost * alloc_global(mass, cost, total, fz)).sum(-1).double()
            prof[bname] = a if bname not in prof else prof[bname] + a
        print(f"# calibration input {tag}: MALA {int((cost * mk).sum()) / (Hq * L):.1f} slots/query",
              file=sys.stderr, flush=True)

    acc = {}
    for tag in evals:
        mk, mass, cost, o, evaluate = instance(tag)
        fz = diagonal_tiles(cost, Bq, Bk, L)
        for bname, total in budgets(mk, cost).items():
            keeps = {
                "static": alloc_within_blocks(mass, cost, static_budget(cost, total, Bq, L), fz),
                "head_position": alloc_within_blocks(mass, cost, profile_budget(prof[bname], cost, total), fz),
                "per_instance_oracle": alloc_global(mass, cost, total, fz),
            }
            if bname == "mala":
                keeps["mala"] = mk
            for name, kp in keeps.items():
                om, out = evaluate(kp)
                a = acc.setdefault(bname, {}).setdefault(name, {"omitted": [], "o_num": 0.0, "o_den": 0.0,
                                                                 "slots": 0})
                a["omitted"].append(om.flatten())
                a["o_num"] += float(((out - o) ** 2).sum())
                a["o_den"] += float((o ** 2).sum())
                a["slots"] += int((cost * kp).sum())
        print(f"# input {tag}: MALA budget {int((cost * mk).sum()) / (Hq * L):.1f} slots/query",
              file=sys.stderr, flush=True)
    rows = {}
    for bname, pols in acc.items():
        rows[bname] = {}
        for name, a in pols.items():
            om = torch.cat(a["omitted"])
            rows[bname][name] = {"omitted_mass_pct": float(om.mean()) * 100,
                                 "omitted_mass_max_pct": float(om.max()) * 100,
                                 "o_rel_l2_pct": (a["o_num"] / a["o_den"]) ** 0.5 * 100,
                                 "slots_per_query": a["slots"] / (len(evals) * Hq * L)}
    out = {
        "metric": "matched-work allocation: omitted mass and O rel-L2 (%) at equal post-score work",
        "value": rows["mala"]["mala"]["omitted_mass_pct"], "unit": "% omitted mass (MALA, at its own work)",
        "higher_is_better": False, "n_gpus": 1, "dtype": "bf16 inputs, fp64 reference", "data": "synthetic",
        "config": {"workload": f"B=1 L={L} Hq={Hq} Hkv={Hkv} d={d} Bq={Bq} Bk={Bk} p={p}, tau={tau}; "
                               f"calibration inputs {calib}, evaluated inputs {evals}"},
        "budgets": rows,
    }
    print(json.dumps(out), flush=True)


def main_tau_sweep(args):
    """Fidelity and cost against tau over the sweep workload (module docstring)."""
    import numpy as np
    import torch

    import adaptive_tile_skipping_amd as mala
    import mala_gen as G

    dev = torch.device("cuda:0")
    torch.cuda.init()
    W = G.WORKLOADS["sweep"]
    Hq, Hkv, d, Bq, Bk = W["Hq"], W["Hkv"], W["d"], W["Bq"], W["Bk"]
    taus = [float(x) for x in args.taus.split(",") if float(x) > 0]
    rows = []
    for L in W["Ls"]:
        inp = G.workload_inputs("sweep", L=L, with_dout=True)
        q, k, v, do = (torch.from_numpy(np.ascontiguousarray(inp[x]).view(np.int16)).view(torch.bfloat16).to(dev)
                       for x in ("q", "k", "v", "dout"))
        o = torch.empty_like(q)
        lse = torch.empty((1, Hq, L), dtype=torch.float32, device=dev)
        ws = mala.fwd_workspace(1, L, Hq, Hkv, d, Bq, Bk, dev)
        bws = mala.bwd_workspace(1, L, Hq, Hkv, d, Bq, Bk, dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        stream = torch.cuda.current_stream(dev)
        nQB = -(-L // Bq)
        n_visit = Hq * sum((min(L, qb * Bq + Bq) - 1) // Bk + 1 for qb in range(nQB))

        def timed(t, n=max(5, args.steps)):
            for _ in range(args.warmup):
                mala.mala_fwd(q, k, v, t, Bq, Bk, o=o, lse=lse, ws=ws)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for e0, e1 in ev:
                e0.record(stream); mala.mala_fwd(q, k, v, t, Bq, Bk, o=o, lse=lse, ws=ws); e1.record(stream)
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

        def timed_bwd(t, o_t, lse_t, n=max(5, args.steps)):
            for _ in range(args.warmup):
                mala.mala_bwd(q, k, v, o_t, do, lse_t, t, Bq, Bk, dq=dq, dk=dk, dv=dv, ws=bws)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for e0, e1 in ev:
                e0.record(stream)
                mala.mala_bwd(q, k, v, o_t, do, lse_t, t, Bq, Bk, dq=dq, dk=dk, dv=dv, ws=bws)
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

        ms0 = timed(0.0)
        o_ref, lse_ref = mala.mala_fwd(q, k, v, 0.0, Bq, Bk, ws=ws)
        bms0 = timed_bwd(0.0, o_ref, lse_ref)
        ref = o_ref.float()
        for t in taus:
            ms = timed(t)
            st = mala.make_stats(1, Hq, L, Bq, Bk, dev, omitted=True)
            ot, lt = mala.mala_fwd(q, k, v, t, Bq, Bk, stats=st, ws=ws)
            torch.cuda.synchronize()
            bms = timed_bwd(t, ot, lt)
            bst = mala.make_stats(1, Hq, L, Bq, Bk, dev)
            mala.mala_bwd(q, k, v, ot, do, lt, t, Bq, Bk, dq=dq, dk=dk, dv=dv, ws=bws, stats=bst)
            torch.cuda.synchronize()
            om = st["omitted_mass"][0].double()                      # [Hq, L]
            err = (ot.float() - ref).double().pow(2).sum(dim=(0, 1, 3)).sqrt()
            nrm = ref.double().pow(2).sum(dim=(0, 1, 3)).sqrt()
            rel = (err / nrm).cpu().numpy()
            rows.append({
                "L": L, "tau": t, "fwd_ms": round(ms, 4), "tau0_fwd_ms": round(ms0, 4),
                "speedup_vs_tau0": round(ms0 / ms, 3),
                "kept_tile_frac": round(int(st["kept_tiles"].sum().item()) / n_visit, 4),
                "slots_per_query": round(float(st["kept_slots"].double().mean().item()), 1),
                "omitted_mean": float(om.mean().item()), "omitted_max": float(om.max().item()),
                "omitted_bound": t / (1 + t),
                "o_rel_l2_per_head": [float(f"{x:.3e}") for x in rel],
                "bwd_ms": round(bms, 4), "tau0_bwd_ms": round(bms0, 4),
                "bwd_kept_tile_frac": round(int(bst["kept_tiles"].sum().item()) / n_visit, 4),
                "bwd_slots_per_query": round(float(bst["kept_slots"].double().mean().item()), 1),
            })
            print(f"# L={L} tau={t}: bwd {bms:.3f} ms (tau=0 {bms0:.3f}), bwd kept {rows[-1]['bwd_kept_tile_frac']}",
                  file=sys.stderr, flush=True)
            print(f"# L={L} tau={t}: {ms:.3f} ms (tau=0 {ms0:.3f}), kept {rows[-1]['kept_tile_frac']}, "
                  f"omitted mean {rows[-1]['omitted_mean']:.2e} max {rows[-1]['omitted_max']:.2e}, "
                  f"O rel-L2 max {rel.max():.2e}", file=sys.stderr, flush=True)
        del q, k, v, do, o, ws, bws, dq, dk, dv
    last = [r for r in rows if r["L"] == W["Ls"][-1] and r["tau"] == 1.0]
    out = {
        "metric": "MALA fidelity vs cost against tau (sweep workload: forward and backward ms, kept tiles, "
                  "slots/query, omitted mass, O rel-L2 vs tau=0)",
        "value": last[0]["speedup_vs_tau0"] if last else None,
        "unit": "forward speedup vs tau=0 at the longest L, tau=1",
        "n_gpus": 1, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"sweep (B=1 Hq={Hq} Hkv={Hkv} d={d} Bq={Bq} Bk={Bk}, KV heads 2-3 diffuse)",
                   "Ls": list(W["Ls"]), "taus": taus},
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(the attention operator shards by heads with no communication; run one process per GPU).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "prefill_128k":
        main_prefill(args)
        return
    if args.workload == "tau_sweep":
        main_tau_sweep(args)
        return
    if args.workload == "matched_work":
        main_matched_work(args)
        return

    import numpy as np
    import torch

    import adaptive_tile_skipping_amd as mala
    import mala_gen as G

    dev = torch.device("cuda:0")
    torch.cuda.init()
    tau = args.tau
    W = G.WORKLOADS["train_128k"]
    B, L, Hq, Hkv, d, Bq, Bk = W["B"], W["L"], W["Hq"], W["Hkv"], W["d"], W["Bq"], W["Bk"]
    WD = G.WORKLOADS["decode_128k"]
    DB, DN, DHq, DHkv, Dd = WD["B"], WD["N"], WD["Hq"], WD["Hkv"], WD["d"]

    t_gen = time.time()
    inp = G.workload_inputs("train_128k")
    dinp = G.workload_inputs("decode_128k")

    def tens(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (tens(inp[x]) for x in ("q", "k", "v", "dout"))
    qd, kc, vc = (tens(dinp[x]) for x in ("q", "k", "v"))
    t_gen = time.time() - t_gen

    # preallocated outputs and workspaces: the timed step allocates nothing
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fws = mala.fwd_workspace(B, L, Hq, Hkv, d, Bq, Bk, dev)
    bws = mala.bwd_workspace(B, L, Hq, Hkv, d, Bq, Bk, dev)
    od = torch.empty_like(qd)
    lsed = torch.empty((DB, DHq), dtype=torch.float32, device=dev)
    keptd = torch.empty((DB, DHkv), dtype=torch.int32, device=dev)
    dws = mala.decode_workspace(DB, DN, DHq, DHkv, Dd, 64, dev)

    def fwd(t):
        mala.mala_fwd(q, k, v, t, Bq, Bk, o=o, lse=lse, ws=fws)

    def bwd(t):
        mala.mala_bwd(q, k, v, o, do, lse, t, Bq, Bk, dq=dq, dk=dk, dv=dv, ws=bws)

    def dec(t):
        mala.mala_decode(qd, kc, vc, t, 64, o=od, lse=lsed, kept_tiles=keptd, ws=dws)

    if args.traffic_probe:
        if args.traffic_probe == "fwd":
            what = "2 x mala_fwd (train_128k, tau=%g)" % tau
            for _ in range(2):
                fwd(tau)
                torch.cuda.synchronize()
        elif args.traffic_probe == "bwd":
            what = "mala_fwd + 2 x mala_bwd (train_128k, tau=%g)" % tau
            fwd(tau)
            for _ in range(2):
                bwd(tau)
                torch.cuda.synchronize()
        else:
            what = "2 x mala_decode (decode_128k, tau=%g), each after a 512 MB read" % tau
            flush = torch.ones(1 << 27, dtype=torch.float32, device=dev)
            for _ in range(2):
                float(flush.sum())
                dec(tau)
                torch.cuda.synchronize()
            del flush
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": what + " + 1 GiB device copy", "copy_bytes": src.numel() * 4}),
              flush=True)
        return

    def timed_steps(t, steps, warmup):
        for _ in range(warmup):
            fwd(t); bwd(t); dec(t)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        peak_base[t] = torch.cuda.memory_allocated(dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        t0 = time.perf_counter()
        for s in range(steps):
            ev[s][0].record(); fwd(t)
            ev[s][1].record(); bwd(t)
            ev[s][2].record(); dec(t)
            ev[s][3].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps * 1e3
        peak_step[t] = torch.cuda.max_memory_allocated(dev)
        f = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        b = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        dd = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
        return wall, f, b, dd

    peak_base, peak_step = {}, {}
    ms_step, fwd_ms, bwd_ms, dec_ms = timed_steps(tau, args.steps, args.warmup)
    print(f"# tau={tau}: step {ms_step:.3f} ms (fwd {fwd_ms:.3f}, bwd {bwd_ms:.3f}, decode {dec_ms * 1e3:.1f} us)",
          file=sys.stderr, flush=True)

    # decode alone with the caches flushed from the 256 MB Infinity Cache: a
    # 512 MB read before each call (a write would leave dirty lines whose
    # write-back to HBM lands inside the timed decode)
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def dec_flushed(t, n=10):
        times = []
        for _ in range(n + 2):
            torch.sum(flush, dim=0, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(); dec(t); e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times[2:]))

    dec_us = dec_flushed(tau) * 1e3

    # the same decode captured once in a HIP graph and replayed (the library
    # enqueues kernels only), flushed the same way before each replay
    def dec_graph_us(t, n=10):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            dec(t)
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            dec(t)
        times = []
        for _ in range(n + 2):
            torch.sum(flush, dim=0, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(); gr.replay(); e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times[2:])) * 1e3

    dec_graph = dec_graph_us(tau)
    res0 = None
    if not args.no_tau0:
        ms0, f0, b0, _ = timed_steps(0.0, max(2, min(args.steps, 3)), 1)
        d0 = dec_flushed(0.0) * 1e3
        res0 = dict(ms_per_step=ms0, fwd_ms=f0, bwd_ms=b0, decode_us=d0)
        print(f"# tau=0: step {ms0:.3f} ms (fwd {f0:.3f}, bwd {b0:.3f}, decode {d0:.1f} us)",
              file=sys.stderr, flush=True)

    # ---- decision statistics of the benchmarked step (untimed)
    fst = mala.make_stats(B, Hq, L, Bq, Bk, dev)
    mala.mala_fwd(q, k, v, tau, Bq, Bk, o=o, lse=lse, stats=fst, ws=fws)
    bst = mala.make_stats(B, Hq, L, Bq, Bk, dev)
    mala.mala_bwd(q, k, v, o, do, lse, tau, Bq, Bk, dq=dq, dk=dk, dv=dv, ws=bws, stats=bst)
    mala.mala_decode(qd, kc, vc, tau, 64, o=od, lse=lsed, kept_tiles=keptd, ws=dws)
    torch.cuda.synchronize()
    nQB, nKT = -(-L // Bq), -(-L // Bk)
    visited = np.array([((min(L, qb * Bq + Bq) - 1) // Bk) + 1 for qb in range(nQB)], dtype=np.int64)
    n_visit = int(visited.sum()) * B * Hq
    kf = int(fst["kept_tiles"].sum().item())
    kb = int(bst["kept_tiles"].sum().item())
    slots_f = float(fst["kept_slots"].double().sum().item())
    slots_b = float(bst["kept_slots"].double().sum().item())
    pairs = B * Hq * L * (L + 1) // 2
    tile_flop = 2.0 * Bq * Bk * d
    dense_fwd = 4.0 * d * pairs
    dense_bwd = 10.0 * d * pairs
    dense_dec = 4.0 * Dd * DN * DHq * DB
    # algorithmic work of each launch (legal slots only)
    alg_fwd = 2.0 * d * pairs + 2.0 * d * slots_f
    alg_bwd = 2.0 * d * pairs + 8.0 * d * slots_b
    # MFMA work the kernels issue (whole tiles): forward QK^T on every visited
    # tile and P.V on kept ones; backward the decision scan on every visited
    # tile (tau > 0 only), then per kept tile S, dP, dV, dK in the dK/dV pass
    # and S, dP, dQ again in the dQ pass
    exec_fwd = tile_flop * (n_visit + kf)
    exec_bwd = tile_flop * ((n_visit if tau > 0 else 0) + 7 * kb)
    kept_dec = int(keptd.sum().item())
    nT = -(-DN // 64)
    dec_bytes = DB * DN * DHkv * Dd * 2 + kept_dec * 64 * Dd * 2      # all of K + the kept V tiles
    dec_bytes0 = 2 * DB * DN * DHkv * Dd * 2
    G_dec = DHq // DHkv
    alg_dec = 2.0 * Dd * DN * DHq * DB + 2.0 * Dd * min(kept_dec * 64, DB * DHkv * DN) * G_dec

    value = (alg_fwd + alg_bwd + alg_dec) / (ms_step * 1e-3) / 1e12

    # ---- what the part sustains, for reading the rates against (after the
    # timed work, so the probes' load does not precede it)
    sustained = measure_sustained(mala, dev, kc, lambda: torch.sum(flush, dim=0, out=sink))
    dense_step = (dense_fwd + dense_bwd + dense_dec) / (ms_step * 1e-3) / 1e12

    # ---- device memory per operator (the library allocates nothing itself:
    # outputs and workspaces are the caller's, allocated once above)
    MiB = 1 << 20
    nbytes = lambda *ts: sum(x.numel() * x.element_size() for x in ts)  # noqa: E731
    memory = {
        "unit": "MiB",
        "inputs": round(nbytes(q, k, v, do, qd, kc, vc) / MiB, 3),
        "fwd": {"outputs": round(nbytes(o, lse) / MiB, 3), "workspace": round(nbytes(fws) / MiB, 3)},
        "bwd": {"outputs": round(nbytes(dq, dk, dv) / MiB, 3), "workspace": round(nbytes(bws) / MiB, 3)},
        "decode": {"outputs": round(nbytes(od, lsed, keptd) / MiB, 3), "workspace": round(nbytes(dws) / MiB, 3)},
        # allocator peak during the timed steps minus what was allocated before them
        "transient_in_step": {f"tau={t:g}": round((peak_step[t] - peak_base[t]) / MiB, 3) for t in peak_step},
        "note": "per rank; the same outputs and workspaces serve tau = 0 and tau > 0, and the library "
                "allocates nothing during a call; the forward workspace is an fp16 copy of V",
    }

    # ---- roofline of the dominant kernel (by measured time)
    cand = {"mala_fwd_kernel": (fwd_ms, alg_fwd), "mala_bwd (pre+scan+gradient+convert)": (bwd_ms, alg_bwd)}
    dom = max(cand, key=lambda n: cand[n][0])
    dms, dflop = cand[dom]
    achieved = dflop / (dms * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic() if dom == "mala_fwd_kernel" else None,
                "algorithmic_tflop_per_launch": round(dflop / 1e12, 3), "launch_ms": round(dms, 4),
                "frac_of_sustained": round(achieved / sustained["mfma_bf16_tflops"], 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "train_128k fwd+bwd (B=1 L=131072 Hq=5 Hkv=1 d=128 Bq=128 Bk=64) + "
                               "decode_128k (B=8 N=131072 Hq=5 Hkv=1 d=128 Bk_dec=64)",
                   "tau": tau},
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "decode_us_in_step": round(dec_ms * 1e3, 2),
        "decode_us": round(dec_us, 2),
        "decode_us_graph": round(dec_graph, 2),
        "decode_tokens_per_s": round(DB / (dec_us * 1e-6), 1),
        "decode_hbm_gbs": round(dec_bytes / (dec_us * 1e-6) / 1e9, 1),
        "value_definition": "algorithmic FLOPs of the step (scores of every legal pair + post-score work of "
                            "retained pairs, fwd + bwd + decode) / step time",
        "algorithmic_tflops": {"fwd": round(alg_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                               "bwd": round(alg_bwd / (bwd_ms * 1e-3) / 1e12, 2)},
        "effective_tflops": {"fwd": round(dense_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                             "bwd": round(dense_bwd / (bwd_ms * 1e-3) / 1e12, 2),
                             "step": round(dense_step, 2)},
        "executed_tflops": {"fwd": round(exec_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                            "bwd": round(exec_bwd / (bwd_ms * 1e-3) / 1e12, 2)},
        "skip": {"fwd_kept_tile_frac": round(kf / n_visit, 4), "bwd_kept_tile_frac": round(kb / n_visit, 4),
                 "decode_kept_tile_frac": round(kept_dec / (DB * DHkv * nT), 4)},
        "slots_per_query": {"fwd": round(slots_f / (B * Hq * L), 1), "bwd": round(slots_b / (B * Hq * L), 1)},
        "roofline": roofline,
        "sustained": sustained,
        "fwd_bwd_executed_tflops": round((exec_fwd + exec_bwd) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2),
        "decode_frac_of_sustained_read": round(dec_bytes / (dec_us * 1e-6) / 1e9 / sustained["hbm_read_gbs"], 4),
        "memory": memory,
        "gen_s": round(t_gen, 1),
    }
    if res0 is not None:
        out["tau0"] = {k2: round(v2, 4) for k2, v2 in res0.items()}
        out["tau0"]["decode_hbm_gbs"] = round(dec_bytes0 / (res0["decode_us"] * 1e-6) / 1e9, 1)
        out["tau0"]["decode_frac_of_sustained_read"] = round(
            dec_bytes0 / (res0["decode_us"] * 1e-6) / 1e9 / sustained["hbm_read_gbs"], 4)
        out["speedup_vs_tau0"] = {"fwd": round(res0["fwd_ms"] / fwd_ms, 3), "bwd": round(res0["bwd_ms"] / bwd_ms, 3),
                                  "decode": round(res0["decode_us"] / dec_us, 3),
                                  "step": round(res0["ms_per_step"] / ms_step, 3)}

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same workload
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args, inp, dinp, W, WD, tau)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
