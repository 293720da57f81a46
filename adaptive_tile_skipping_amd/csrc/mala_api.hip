// libmala C ABI: argument validation on the host, then kernel launches on the
// caller's stream.  Nothing is enqueued when validation fails.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/mala.h"
#include "mala_internal.h"

using namespace mala;

// Device scratch of mala_decode_noalloc, for callers that cannot allocate.
// Each GPU holds its own copy for the life of the process.  Host code never
// passes `scratch` itself (its host-side name is only a handle): the address
// on each device comes from hipGetSymbolAddress, looked up once per device
// with that device current, and kept in scratch_addr[].
static __device__ __align__(256) unsigned char scratch[MALA_DECODE_NOALLOC_MAX_BYTES];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool t4_ok(const mala_t4& t, bool need) {
    if (!t.ptr) return !need;
    if (!aligned16(t.ptr)) return false;
    if ((t.sb % 8) || (t.sl % 8) || (t.sh % 8)) return false;
    if (t.sb < 0 || t.sl < 0 || t.sh < 0) return false;
    return true;
}

bool tau_ok(float tau) { return isfinite(tau) && tau >= 0.f; }

float log2_tau(float tau) { return tau == 0.f ? -INFINITY : (float)log2((double)tau); }

bool fwd_shape_supported(int d, int Bq, int Bk) {
    return (d == 128 && Bq == 128 && Bk == 64) || (d == 64 && Bq == 64 && Bk == 64);
}

bool dims_ok(int B, int L, int Hq, int Hkv, int d) {
    if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return false;
    if (Hq % Hkv) return false;
    if ((int64_t)L * Hq * B > INT32_MAX / 2) return false;
    return true;
}

// Workgroups per XCD run in groups of `chunk` consecutive units: one query
// block of every q head of a KV head, twice, so that the heads sharing K/V
// tiles sit on the same L2.
int pick_chunk(int Hq, int Hkv) {
    const int G = Hq / Hkv;
    int c = 2 * G;
    if (c < 4) c = 4;
    if (c > 32) c = 32;
    return c;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units of the current device, for the persistent forward launch
// (cached per device; concurrent first calls store the same value).
int device_cus() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cached[dev] = n;
    return n;
}

// Decode splits per (sequence, KV head) of the tau = 0 path, one wave each:
// enough waves (~2048) to keep many cache loads in flight, no more splits
// with tiles than the cache has tiles, rounded up to whole workgroups of 8.
void decode_split(int B, int Hkv, int nT, int* nsplit, int* tps) {
    const int ngrp = B * Hkv;
    int ns = (2048 + ngrp - 1) / ngrp;
    if (ns > 512) ns = 512;
    if (ns > nT) ns = nT;
    if (ns < 1) ns = 1;
    int t = (nT + ns - 1) / ns;
    ns = (nT + t - 1) / t;
    *nsplit = (ns + 7) / 8 * 8;         // whole workgroups of 8 splits (the extra ones are empty)
    *tps = t;
}

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];

// This device's address of `scratch` (nullptr on failure).  Concurrent first
// calls on one device look it up twice and store the same value.
void* device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* ptr = scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_addr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

// P.V workgroups of the tau > 0 decode: persistent, two per CU at most; the
// kept tiles of all groups are split evenly over them on the device.
int decode_pv_workgroups(int B, int Hkv, int nT) {
    const int64_t tiles = (int64_t)B * Hkv * nT;
    return (int)(tiles < 512 ? (tiles < 1 ? 1 : tiles) : 512);
}

}  // namespace

extern "C" {

const char* mala_status_string(mala_status s) {
    switch (s) {
        case MALA_OK: return "MALA_OK";
        case MALA_ERR_INVALID_ARG: return "MALA_ERR_INVALID_ARG";
        case MALA_ERR_UNSUPPORTED: return "MALA_ERR_UNSUPPORTED";
        case MALA_ERR_WORKSPACE: return "MALA_ERR_WORKSPACE";
        case MALA_ERR_HIP: return "MALA_ERR_HIP";
    }
    return "MALA_ERR_UNKNOWN";
}

const char* mala_version(void) { return "0.1.0 gfx950"; }

size_t mala_fwd_workspace_size(int B, int L, int Hq, int Hkv, int d, int Bq, int Bk) {
    if (!dims_ok(B, L, Hq, Hkv, d) || !fwd_shape_supported(d, Bq, Bk)) return 0;
    const size_t Lpad = (size_t)((L + Bk - 1) / Bk) * Bk;
    return align256((size_t)B * Hkv * Lpad * d * 2) + 256;      // fp16 V copy, work queues
}

mala_status mala_fwd(mala_t4 q, mala_t4 k, mala_t4 v, int B, int L, int Hq, int Hkv, int d,
                     float tau, int Bq, int Bk, mala_t4 o, float* lse,
                     const mala_tile_stats* stats, void* ws, size_t ws_bytes, void* stream) {
    if (!dims_ok(B, L, Hq, Hkv, d) || !tau_ok(tau)) return MALA_ERR_INVALID_ARG;
    if (!t4_ok(q, true) || !t4_ok(k, true) || !t4_ok(v, true) || !t4_ok(o, true) || !lse)
        return MALA_ERR_INVALID_ARG;
    if (!fwd_shape_supported(d, Bq, Bk)) return MALA_ERR_UNSUPPORTED;
    // one KV head's keys and its fp16 V copy are addressed through 32-bit buffer ranges
    if (((int64_t)(L - 1) * k.sl + d) * 2 > INT32_MAX || (int64_t)(L + Bq) * d * 2 > INT32_MAX)
        return MALA_ERR_UNSUPPORTED;
    const size_t need = mala_fwd_workspace_size(B, L, Hq, Hkv, d, Bq, Bk);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return MALA_ERR_WORKSPACE;
    FwdParams p;
    memset(&p, 0, sizeof(p));
    p.q = (const uint16_t*)q.ptr; p.k = (const uint16_t*)k.ptr; p.v = (const uint16_t*)v.ptr;
    p.o = (uint16_t*)o.ptr; p.lse = lse;
    p.q_sb = q.sb; p.q_sl = q.sl; p.q_sh = q.sh;
    p.k_sb = k.sb; p.k_sl = k.sl; p.k_sh = k.sh;
    p.v_sb = v.sb; p.v_sl = v.sl; p.v_sh = v.sh;
    p.o_sb = o.sb; p.o_sl = o.sl; p.o_sh = o.sh;
    p.B = B; p.L = L; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.nQB = (L + Bq - 1) / Bq; p.nKT = (L + Bk - 1) / Bk;
    p.nunits = B * Hq * p.nQB;
    p.chunk = pick_chunk(Hq, Hkv);
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    p.log2_tau = log2_tau(tau);
    p.nwords = (p.nKT + 31) / 32;
    p.vh = (uint16_t*)ws;
    p.Lpad = p.nKT * Bk;
    p.queue = (int*)((char*)ws + need - 256);
    p.ncu = device_cus();
    bool st = false;
    if (stats) {
        p.kept_tiles = stats->kept_tiles;
        p.kept_slots = stats->kept_slots;
        p.omitted = stats->omitted_mass;
        p.bits = stats->decision_bits;
        st = stats->omitted_mass != nullptr;
    }
    hipError_t e = launch_fwd(p, d, Bq, Bk, st, (hipStream_t)stream);
    return e == hipSuccess ? MALA_OK : MALA_ERR_HIP;
}

size_t mala_fwd_varlen_workspace_size(int B, int total_k, int Hkv, int d, int Bq, int Bk) {
    if (B <= 0 || total_k < 0 || Hkv <= 0 || !fwd_shape_supported(d, Bq, Bk)) return 0;
    return align256(((size_t)total_k + (size_t)B * Bk) * Hkv * d * 2) + 256;   // fp16 V copy, work queues
}

mala_status mala_fwd_varlen(mala_t3 q, mala_t3 k, mala_t3 v, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int B, int total_q, int total_k, int max_seqlen_q,
                            int max_seqlen_k, int Hq, int Hkv, int d, float tau, int Bq, int Bk, mala_t3 o,
                            float* lse, const mala_tile_stats* stats, void* ws, size_t ws_bytes, void* stream) {
    if (B <= 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return MALA_ERR_INVALID_ARG;
    if (Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv || !tau_ok(tau)) return MALA_ERR_INVALID_ARG;
    if (max_seqlen_q > max_seqlen_k || max_seqlen_q > total_q || max_seqlen_k > total_k) return MALA_ERR_INVALID_ARG;
    if (!cu_seqlens_q || !cu_seqlens_k || !lse) return MALA_ERR_INVALID_ARG;
    if (!t4_ok({q.ptr, 0, q.sl, q.sh}, true) || !t4_ok({k.ptr, 0, k.sl, k.sh}, true) ||
        !t4_ok({v.ptr, 0, v.sl, v.sh}, true) || !t4_ok({o.ptr, 0, o.sl, o.sh}, true))
        return MALA_ERR_INVALID_ARG;
    if ((int64_t)total_q * Hq > INT32_MAX / 2 || (int64_t)total_k + (int64_t)B * Bk > INT32_MAX / 2)
        return MALA_ERR_INVALID_ARG;
    if (!fwd_shape_supported(d, Bq, Bk) || B > 65535) return MALA_ERR_UNSUPPORTED;
    // one sequence's keys of a KV head and its fp16 V copy are addressed through 32-bit buffer ranges
    const int64_t mk = max_seqlen_k > 0 ? max_seqlen_k : 1;
    if (((mk - 1) * k.sl + d) * 2 > INT32_MAX || (mk + Bk) * d * 2 > INT32_MAX) return MALA_ERR_UNSUPPORTED;
    const size_t need = mala_fwd_varlen_workspace_size(B, total_k, Hkv, d, Bq, Bk);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return MALA_ERR_WORKSPACE;
    if (total_q == 0) return MALA_OK;      // no query rows: nothing to compute or write
    FwdParams p;
    memset(&p, 0, sizeof(p));
    p.q = (const uint16_t*)q.ptr; p.k = (const uint16_t*)k.ptr; p.v = (const uint16_t*)v.ptr;
    p.o = (uint16_t*)o.ptr; p.lse = lse;
    p.q_sl = q.sl; p.q_sh = q.sh; p.k_sl = k.sl; p.k_sh = k.sh;
    p.v_sl = v.sl; p.v_sh = v.sh; p.o_sl = o.sl; p.o_sh = o.sh;
    p.B = B; p.L = 0; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
    p.total_q = total_q; p.total_k = total_k; p.max_q = max_seqlen_q; p.max_k = max_seqlen_k;
    p.nQB = max_seqlen_q > 0 ? (max_seqlen_q + Bq - 1) / Bq : 1;
    p.nKT = max_seqlen_k > 0 ? (max_seqlen_k + Bk - 1) / Bk : 1;
    p.nunits = B * Hq * p.nQB;
    p.chunk = pick_chunk(Hq, Hkv);
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    p.log2_tau = log2_tau(tau);
    p.nwords = (p.nKT + 31) / 32;
    p.vh = (uint16_t*)ws;
    p.Rk = total_k + B * Bk;
    p.queue = (int*)((char*)ws + need - 256);
    p.ncu = device_cus();
    bool st = false;
    if (stats) {
        p.kept_tiles = stats->kept_tiles;
        p.kept_slots = stats->kept_slots;
        p.omitted = stats->omitted_mass;
        p.bits = stats->decision_bits;
        st = stats->omitted_mass != nullptr;
    }
    hipError_t e = launch_fwd(p, d, Bq, Bk, st, (hipStream_t)stream);
    return e == hipSuccess ? MALA_OK : MALA_ERR_HIP;
}

size_t mala_bwd_workspace_size(int B, int L, int Hq, int Hkv, int d, int Bq, int Bk) {
    if (!dims_ok(B, L, Hq, Hkv, d) || !fwd_shape_supported(d, Bq, Bk)) return 0;
    const size_t Lpad = (size_t)((L + Bq - 1) / Bq) * Bq;
    const size_t prow = (size_t)B * Hq * Lpad;
    const size_t nQB = Lpad / Bq, nKT = (size_t)(L + Bk - 1) / Bk;
    const size_t nwT = ((size_t)(Hq / Hkv) * nQB + 31) / 32;
    const size_t tb = (size_t)B * Hkv * nKT * nwT * sizeof(uint32_t);
    const size_t qbb = (size_t)B * Hq * nQB * ((nKT + 31) / 32) * sizeof(uint32_t);
    return 2 * align256(prow * sizeof(float)) + align256(tb) + align256(qbb);
}

mala_status mala_bwd(mala_t4 q, mala_t4 k, mala_t4 v, mala_t4 o, mala_t4 dout, const float* lse,
                     int B, int L, int Hq, int Hkv, int d, float tau, int Bq, int Bk,
                     mala_t4 dq, mala_t4 dk, mala_t4 dv, void* ws, size_t ws_bytes,
                     const mala_tile_stats* bwd_stats, void* stream) {
    if (!dims_ok(B, L, Hq, Hkv, d) || !tau_ok(tau)) return MALA_ERR_INVALID_ARG;
    if (!t4_ok(q, true) || !t4_ok(k, true) || !t4_ok(v, true) || !t4_ok(o, true) || !t4_ok(dout, true) ||
        !t4_ok(dq, true) || !t4_ok(dk, true) || !t4_ok(dv, true) || !lse)
        return MALA_ERR_INVALID_ARG;
    if (bwd_stats && bwd_stats->omitted_mass) return MALA_ERR_INVALID_ARG;
    if (!fwd_shape_supported(d, Bq, Bk)) return MALA_ERR_UNSUPPORTED;
    // a query block is read through one buffer resource (32-bit byte range)
    if (((int64_t)Bq * q.sl + d) * 2 > INT32_MAX || ((int64_t)(L - 1) * k.sl + d) * 2 > INT32_MAX ||
        ((int64_t)(L - 1) * v.sl + d) * 2 > INT32_MAX)
        return MALA_ERR_UNSUPPORTED;
    const size_t need = mala_bwd_workspace_size(B, L, Hq, Hkv, d, Bq, Bk);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return MALA_ERR_WORKSPACE;
    BwdParams p;
    memset(&p, 0, sizeof(p));
    p.q = (const uint16_t*)q.ptr; p.k = (const uint16_t*)k.ptr; p.v = (const uint16_t*)v.ptr;
    p.o = (const uint16_t*)o.ptr; p.dout = (const uint16_t*)dout.ptr; p.lse = lse;
    p.dq = (uint16_t*)dq.ptr; p.dk = (uint16_t*)dk.ptr; p.dv = (uint16_t*)dv.ptr;
    char* w = (char*)ws;
    p.Lpad = ((L + Bq - 1) / Bq) * Bq;
    const size_t prow = (size_t)B * Hq * p.Lpad;
    p.rowd = (float*)w; w += align256(prow * sizeof(float));
    p.rowc = (float*)w; w += align256(prow * sizeof(float));
    p.tbits = (uint32_t*)w;
    {
        const size_t nQB_ = (size_t)((L + Bq - 1) / Bq), nKT_ = (size_t)((L + Bk - 1) / Bk);
        const size_t nwT_ = ((size_t)(Hq / Hkv) * nQB_ + 31) / 32;
        w += align256((size_t)B * Hkv * nKT_ * nwT_ * sizeof(uint32_t));
    }
    p.qbits = (uint32_t*)w;
    p.q_sb = q.sb; p.q_sl = q.sl; p.q_sh = q.sh;
    p.k_sb = k.sb; p.k_sl = k.sl; p.k_sh = k.sh;
    p.v_sb = v.sb; p.v_sl = v.sl; p.v_sh = v.sh;
    p.o_sb = o.sb; p.o_sl = o.sl; p.o_sh = o.sh;
    p.do_sb = dout.sb; p.do_sl = dout.sl; p.do_sh = dout.sh;
    p.dq_sb = dq.sb; p.dq_sl = dq.sl; p.dq_sh = dq.sh;
    p.dk_sb = dk.sb; p.dk_sl = dk.sl; p.dk_sh = dk.sh;
    p.dv_sb = dv.sb; p.dv_sl = dv.sl; p.dv_sh = dv.sh;
    p.B = B; p.L = L; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.nQB = (L + Bq - 1) / Bq; p.nKT = (L + Bk - 1) / Bk;
    p.chunk = 4;
    p.nwT = (p.G * p.nQB + 31) / 32;
    p.nslab = (L + 255) / 256;
    p.nunits_scan = p.nslab * B * Hq;
    p.chunk_scan = pick_chunk(Hq, Hkv);
    p.nunits_dq = B * Hq * p.nQB;
    p.chunk_dq = pick_chunk(Hq, Hkv);
    p.ncu = device_cus();
    p.scale = (float)(1.0 / sqrt((double)d));
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    p.log2_tau = log2_tau(tau);
    p.nwords = (p.nKT + 31) / 32;
    if (bwd_stats) {
        p.kept_tiles = bwd_stats->kept_tiles;
        p.kept_slots = bwd_stats->kept_slots;
        p.bits = bwd_stats->decision_bits;
    }
    hipError_t e = launch_bwd(p, d, Bq, Bk, (hipStream_t)stream);
    return e == hipSuccess ? MALA_OK : MALA_ERR_HIP;
}

size_t mala_bwd_varlen_workspace_size(int B, int total_q, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv,
                                      int d, int Bq, int Bk) {
    if (B <= 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv ||
        !fwd_shape_supported(d, Bq, Bk))
        return 0;
    const size_t prow = (size_t)Hq * ((size_t)total_q + (size_t)B * Bq);
    const size_t nQB = max_seqlen_q > 0 ? (size_t)(max_seqlen_q + Bq - 1) / Bq : 1;
    const size_t nKT = max_seqlen_k > 0 ? (size_t)(max_seqlen_k + Bk - 1) / Bk : 1;
    const size_t nwT = ((size_t)(Hq / Hkv) * nQB + 31) / 32;
    const size_t tb = (size_t)B * Hkv * nKT * nwT * sizeof(uint32_t);
    const size_t qbb = (size_t)B * Hq * nQB * ((nKT + 31) / 32) * sizeof(uint32_t);
    return 2 * align256(prow * sizeof(float)) + align256(tb) + align256(qbb);
}

mala_status mala_bwd_varlen(mala_t3 q, mala_t3 k, mala_t3 v, mala_t3 o, mala_t3 dout, const float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int total_q,
                            int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d, float tau,
                            int Bq, int Bk, mala_t3 dq, mala_t3 dk, mala_t3 dv, void* ws, size_t ws_bytes,
                            const mala_tile_stats* bwd_stats, void* stream) {
    if (B <= 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return MALA_ERR_INVALID_ARG;
    if (Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv || !tau_ok(tau)) return MALA_ERR_INVALID_ARG;
    if (max_seqlen_q > max_seqlen_k || max_seqlen_q > total_q || max_seqlen_k > total_k) return MALA_ERR_INVALID_ARG;
    if (!cu_seqlens_q || !cu_seqlens_k || !lse) return MALA_ERR_INVALID_ARG;
    const mala_t3 ts[8] = {q, k, v, o, dout, dq, dk, dv};
    for (const mala_t3& t : ts)
        if (!t4_ok({t.ptr, 0, t.sl, t.sh}, true)) return MALA_ERR_INVALID_ARG;
    if (bwd_stats && bwd_stats->omitted_mass) return MALA_ERR_INVALID_ARG;
    if ((int64_t)total_q * Hq > INT32_MAX / 2 || (int64_t)total_k * Hkv > INT32_MAX / 2 ||
        (int64_t)total_q + (int64_t)B * Bq > INT32_MAX / 2)
        return MALA_ERR_INVALID_ARG;
    if (!fwd_shape_supported(d, Bq, Bk) || B > 65535) return MALA_ERR_UNSUPPORTED;
    // a query block and one sequence's keys are read through 32-bit buffer ranges
    const int64_t mk = max_seqlen_k > 0 ? max_seqlen_k : 1;
    if (((int64_t)Bq * q.sl + d) * 2 > INT32_MAX || ((int64_t)Bq * dout.sl + d) * 2 > INT32_MAX ||
        ((mk - 1) * k.sl + d) * 2 > INT32_MAX || ((mk - 1) * v.sl + d) * 2 > INT32_MAX)
        return MALA_ERR_UNSUPPORTED;
    const size_t need = mala_bwd_varlen_workspace_size(B, total_q, max_seqlen_q, max_seqlen_k, Hq, Hkv, d, Bq, Bk);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return MALA_ERR_WORKSPACE;
    if (total_k == 0) return MALA_OK;      // no keys, so no queries either: nothing to write
    BwdParams p;
    memset(&p, 0, sizeof(p));
    p.q = (const uint16_t*)q.ptr; p.k = (const uint16_t*)k.ptr; p.v = (const uint16_t*)v.ptr;
    p.o = (const uint16_t*)o.ptr; p.dout = (const uint16_t*)dout.ptr; p.lse = lse;
    p.dq = (uint16_t*)dq.ptr; p.dk = (uint16_t*)dk.ptr; p.dv = (uint16_t*)dv.ptr;
    p.q_sl = q.sl; p.q_sh = q.sh; p.k_sl = k.sl; p.k_sh = k.sh; p.v_sl = v.sl; p.v_sh = v.sh;
    p.o_sl = o.sl; p.o_sh = o.sh; p.do_sl = dout.sl; p.do_sh = dout.sh;
    p.dq_sl = dq.sl; p.dq_sh = dq.sh; p.dk_sl = dk.sl; p.dk_sh = dk.sh; p.dv_sl = dv.sl; p.dv_sh = dv.sh;
    p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
    p.total_q = total_q; p.total_k = total_k; p.max_q = max_seqlen_q; p.max_k = max_seqlen_k;
    p.Rq = total_q + B * Bq;
    p.B = B; p.L = 0; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv;
    p.nQB = max_seqlen_q > 0 ? (max_seqlen_q + Bq - 1) / Bq : 1;
    p.nKT = max_seqlen_k > 0 ? (max_seqlen_k + Bk - 1) / Bk : 1;
    p.Lpad = p.nQB * Bq;
    char* w = (char*)ws;
    const size_t prow = (size_t)Hq * p.Rq;
    p.rowd = (float*)w; w += align256(prow * sizeof(float));
    p.rowc = (float*)w; w += align256(prow * sizeof(float));
    p.nwT = (p.G * p.nQB + 31) / 32;
    p.tbits = (uint32_t*)w; w += align256((size_t)B * Hkv * p.nKT * p.nwT * sizeof(uint32_t));
    p.qbits = (uint32_t*)w;
    p.chunk = 4;
    p.nslab = (p.nQB * Bq + 255) / 256;
    p.nunits_scan = p.nslab * B * Hq;
    p.chunk_scan = pick_chunk(Hq, Hkv);
    p.nunits_dq = B * Hq * p.nQB;
    p.chunk_dq = pick_chunk(Hq, Hkv);
    p.ncu = device_cus();
    p.scale = (float)(1.0 / sqrt((double)d));
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    p.log2_tau = log2_tau(tau);
    p.nwords = (p.nKT + 31) / 32;
    if (bwd_stats) {
        p.kept_tiles = bwd_stats->kept_tiles;
        p.kept_slots = bwd_stats->kept_slots;
        p.bits = bwd_stats->decision_bits;
    }
    hipError_t e = launch_bwd(p, d, Bq, Bk, (hipStream_t)stream);
    return e == hipSuccess ? MALA_OK : MALA_ERR_HIP;
}

size_t mala_decode_workspace_size(int B, int N, int Hq, int Hkv, int d, int Bk_dec) {
    if (!dims_ok(B, N, Hq, Hkv, d) || (d != 128 && d != 64) || Bk_dec != 64) return 0;
    const int G = Hq / Hkv;
    const size_t nT = (size_t)(N + Bk_dec - 1) / Bk_dec;
    const size_t grp = (size_t)B * Hkv;
    int ns, tps;
    decode_split(B, Hkv, (int)nT, &ns, &tps);
    const size_t nsplit = (size_t)ns;
    const size_t npv = decode_pv_workgroups(B, Hkv, (int)nT);
    const size_t nslot = grp * nsplit > npv + grp ? grp * nsplit : npv + grp;
    size_t s = 0;
    s += 2 * align256(grp * G * ((nT + 3) / 4 * 4) * sizeof(float));   // tmax, tsum
    s += align256(grp * nT * G * Bk_dec * sizeof(uint16_t));   // spill
    s += align256(grp * nT * sizeof(int32_t));                // klist
    s += align256(grp * sizeof(int32_t));                     // kcount
    s += align256(grp * G * sizeof(float));                   // lse2
    s += align256(grp * 2 * sizeof(int32_t));                 // pvinfo
    s += align256(nslot * G * d * sizeof(float));             // part_o
    s += align256(grp * nsplit * G * 2 * sizeof(float));      // part_ml
    return s;
}

}  // extern "C"

namespace {
mala_status decode_impl(const void* q, mala_t4 kcache, mala_t4 vcache, const int32_t* seqlens, int B, int N,
                        int Hq, int Hkv, int d, float tau, int Bk_dec, void* o, float* lse, int32_t* kept_tiles,
                        uint32_t* decision_bits, void* ws, size_t ws_bytes, void* stream) {
    if (!dims_ok(B, N, Hq, Hkv, d) || !tau_ok(tau)) return MALA_ERR_INVALID_ARG;
    if (!q || !aligned16(q) || !o || !aligned16(o) || !lse) return MALA_ERR_INVALID_ARG;
    if (!t4_ok(kcache, true) || !t4_ok(vcache, true)) return MALA_ERR_INVALID_ARG;
    if ((d != 128 && d != 64) || Bk_dec != 64) return MALA_ERR_UNSUPPORTED;
    const int G = Hq / Hkv;
    if (G > 16) return MALA_ERR_UNSUPPORTED;
    const size_t need = mala_decode_workspace_size(B, N, Hq, Hkv, d, Bk_dec);
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return MALA_ERR_WORKSPACE;
    DecParams p;
    memset(&p, 0, sizeof(p));
    p.q = (const uint16_t*)q; p.k = (const uint16_t*)kcache.ptr; p.v = (const uint16_t*)vcache.ptr;
    p.o = (uint16_t*)o; p.lse = lse; p.kept_tiles = kept_tiles; p.bits = decision_bits;
    p.seqlens = seqlens;
    p.k_sb = kcache.sb; p.k_sl = kcache.sl; p.k_sh = kcache.sh;
    p.v_sb = vcache.sb; p.v_sl = vcache.sl; p.v_sh = vcache.sh;
    p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.G = G;
    p.nT = (N + Bk_dec - 1) / Bk_dec;
    p.nwords = (p.nT + 31) / 32;
    decode_split(B, Hkv, p.nT, &p.nsplit, &p.tiles_per_split);
    p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    p.log2_tau = log2_tau(tau);
    p.log2_N = (float)log2((double)N);
    const size_t nT = (size_t)p.nT, grp = (size_t)B * Hkv;
    char* w = (char*)ws;
    p.nTp = (p.nT + 3) / 4 * 4;
    p.tmax = (float*)w; w += align256(grp * G * (size_t)p.nTp * sizeof(float));
    p.tsum = (float*)w; w += align256(grp * G * (size_t)p.nTp * sizeof(float));
    p.spill = (uint16_t*)w; w += align256(grp * nT * G * Bk_dec * sizeof(uint16_t));
    p.klist = (int32_t*)w; w += align256(grp * nT * sizeof(int32_t));
    p.kcount = (int32_t*)w; w += align256(grp * sizeof(int32_t));
    p.lse2 = (float*)w; w += align256(grp * G * sizeof(float));
    p.pvinfo = (int32_t*)w; w += align256(grp * 2 * sizeof(int32_t));
    p.npart = p.nsplit / 8;              // dense path: one partial per workgroup of 8 splits
    p.npv = decode_pv_workgroups(B, Hkv, p.nT);
    const size_t nslot = grp * (size_t)p.nsplit > (size_t)p.npv + grp ? grp * (size_t)p.nsplit : (size_t)p.npv + grp;
    p.part_o = (float*)w; w += align256(nslot * G * d * sizeof(float));
    p.part_ml = (float*)w;
    hipError_t e = launch_decode(p, d, Bk_dec, tau == 0.f, (hipStream_t)stream);
    return e == hipSuccess ? MALA_OK : MALA_ERR_HIP;
}
}  // namespace

extern "C" {

mala_status mala_decode(const void* q, mala_t4 kcache, mala_t4 vcache, int B, int N, int Hq, int Hkv,
                        int d, float tau, int Bk_dec, void* o, float* lse, int32_t* kept_tiles,
                        uint32_t* decision_bits, void* ws, size_t ws_bytes, void* stream) {
    return decode_impl(q, kcache, vcache, nullptr, B, N, Hq, Hkv, d, tau, Bk_dec, o, lse, kept_tiles, decision_bits,
                       ws, ws_bytes, stream);
}

mala_status mala_decode_noalloc(const void* q, mala_t4 kcache, mala_t4 vcache, int B, int N, int Hq, int Hkv,
                                int d, float tau, int Bk_dec, void* o, float* lse, int32_t* kept_tiles,
                                uint32_t* decision_bits, void* stream) {
    const size_t need = mala_decode_workspace_size(B, N, Hq, Hkv, d, Bk_dec);
    if (need == 0 || need > (size_t)MALA_DECODE_NOALLOC_MAX_BYTES) {
        // reports the argument error if there is one, else MALA_ERR_WORKSPACE;
        // with no workspace nothing is enqueued
        return decode_impl(q, kcache, vcache, nullptr, B, N, Hq, Hkv, d, tau, Bk_dec, o, lse, kept_tiles,
                           decision_bits, nullptr, 0, stream);
    }
    void* ws = device_scratch();
    if (!ws) return MALA_ERR_HIP;
    return decode_impl(q, kcache, vcache, nullptr, B, N, Hq, Hkv, d, tau, Bk_dec, o, lse, kept_tiles, decision_bits,
                       ws, (size_t)MALA_DECODE_NOALLOC_MAX_BYTES, stream);
}

mala_status mala_decode_varlen(const void* q, mala_t4 kcache, mala_t4 vcache, const int32_t* cache_seqlens, int B,
                               int N, int Hq, int Hkv, int d, float tau, int Bk_dec, void* o, float* lse,
                               int32_t* kept_tiles, uint32_t* decision_bits, void* ws, size_t ws_bytes,
                               void* stream) {
    if (!cache_seqlens) return MALA_ERR_INVALID_ARG;
    return decode_impl(q, kcache, vcache, cache_seqlens, B, N, Hq, Hkv, d, tau, Bk_dec, o, lse, kept_tiles,
                       decision_bits, ws, ws_bytes, stream);
}

}  // extern "C"
