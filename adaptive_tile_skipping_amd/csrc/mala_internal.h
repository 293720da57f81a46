// Host-side kernel parameter blocks and launchers of libmala (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mala {

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int64_t q_sb, q_sl, q_sh, k_sb, k_sl, k_sh, v_sb, v_sl, v_sh, o_sb, o_sl, o_sh;
    int B, L, Hq, Hkv, G, nQB, nKT, nunits, chunk;
    float scale_log2;   // log2(e) / sqrt(d): scores in base 2
    float log2_tau;     // log2(tau); -inf for tau = 0
    int32_t* kept_tiles;
    int32_t* kept_slots;
    float* omitted;
    uint32_t* bits;
    int nwords;
    uint16_t* vh;       // fp16 copy of V (workspace): B x Hkv x Lpad keys, or Hkv x Rk packed,
                        // as transposed [d][Bk] tiles
    int Lpad;           // nKT * Bk
    // packed variable-length batches (cu_q == nullptr: the fixed-length layout
    // above, with q/k/v/o strides sb, sl, sh and lse [B, Hq, L])
    const int32_t* cu_q;   // [B + 1] device: first query row of each sequence
    const int32_t* cu_k;   // [B + 1] device: first key row of each sequence
    int total_q, total_k;  // packed rows; lse / kept_slots / omitted are [Hq, total_q]
    int max_q, max_k;      // longest query and key counts (nQB, nKT derive from them)
    int Rk;                // total_k + B * Bk: V copy rows per KV head (sequence b at cu_k[b] + b Bk)
    int* queue;            // [8] work queues of the forward kernel (workspace; zeroed by the V copy)
    int ncu;               // compute units of the device (persistent forward workgroups per CU follow)
};

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* rowd;        // [B, Hq, Lpad] fp32: D_i = dO_i . O_i (0 past L)
    float* rowc;        // [B, Hq, Lpad] fp32: LSE_i * log2(e) (0 past L)
    uint32_t* tbits;    // [B, Hkv, nKT, nwT] bit (h % G) * nQB + qb: tile (qb, kt) of q head h kept
    uint32_t* qbits;    // [B, Hq, nQB, nwords] bit kt: the same tile, query-major
    int Lpad;           // nQB * Bq
    int64_t q_sb, q_sl, q_sh, k_sb, k_sl, k_sh, v_sb, v_sl, v_sh, o_sb, o_sl, o_sh;
    int64_t do_sb, do_sl, do_sh, dq_sb, dq_sl, dq_sh, dk_sb, dk_sl, dk_sh, dv_sb, dv_sl, dv_sh;
    int B, L, Hq, Hkv, G, nQB, nKT, chunk;       // chunk: adjacent dK/dV units per XCD
    int nwT;            // ceil(G * nQB / 32)
    int nslab, nunits_scan, chunk_scan;   // scan kernel: 256-query slabs, work units
    int nunits_dq, chunk_dq;              // dQ pass: (batch, q head, query block) units
    int ncu;            // compute units of the device
    float scale;        // 1 / sqrt(d)
    float scale_log2;   // log2(e) / sqrt(d)
    float log2_tau;
    int32_t* kept_tiles;
    int32_t* kept_slots;
    uint32_t* bits;
    int nwords;
    // packed variable-length batches (cu_q == nullptr: the fixed-length layout
    // with strides sb, sl, sh, lse [B, Hq, L] and row terms [B, Hq, Lpad])
    const int32_t* cu_q;   // [B + 1] device: first query row of each sequence
    const int32_t* cu_k;   // [B + 1] device: first key row of each sequence
    int total_q, total_k;  // packed rows; lse / kept_slots are [Hq, total_q]
    int max_q, max_k;      // longest query and key counts (nQB, nKT derive from them)
    int Rq;                // total_q + B * Bq: row-term rows per q head (sequence b at cu_q[b] + b Bq)
};

struct DecParams {
    const uint16_t* q;      // [B, Hq, d]
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;            // [B, Hq, d]
    float* lse;             // [B, Hq]
    int32_t* kept_tiles;    // [B, Hkv] or null
    uint32_t* bits;         // [B, Hkv, nwords] or null
    int nwords;
    int64_t k_sb, k_sl, k_sh, v_sb, v_sl, v_sh;
    int B, N, Hq, Hkv, G, nT, nsplit, tiles_per_split;
    int npart;              // dense path: partials per (sequence, KV head), one per workgroup of 8 splits
    int npv;                // P.V workgroups (tau > 0)
    float scale_log2;
    float log2_tau;
    float log2_N;
    const int32_t* seqlens; // [B] device cache lengths (1 .. N), or null: every sequence has N keys
    // workspace
    float* tmax;            // [B, Hkv, G, nTp] tile row max (base 2); nTp = nT rounded up to 4
    float* tsum;            // [B, Hkv, G, nTp] sum 2^(s - tile max)
    int nTp;
    uint16_t* spill;        // [B, Hkv, nT, G, 64] fp16 2^(score - tile max), tile-major
    int32_t* klist;         // [B, Hkv, nT]     retained tiles, newest first
    int32_t* kcount;        // [B, Hkv]
    float* lse2;            // [B, Hkv, G]      base-2 final log-normaliser
    int32_t* pvinfo;        // [B, Hkv, 2] first P.V workgroup and slot count of each group's partials
    float* part_o;          // dense: [B, Hkv, npart, G, d] partial outputs; tau > 0: [npv + B Hkv, G, d]
                            // (slot workgroup + group)
    float* part_ml;         // [B, Hkv, nsplit, G, 2] partial (max, sum) (dense path)
};

hipError_t launch_fwd(const FwdParams& p, int d, int Bq, int Bk, bool stats, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int d, int Bq, int Bk, hipStream_t s);
hipError_t launch_decode(const DecParams& p, int d, int Bkd, bool dense, hipStream_t s);

}  // namespace mala
