// MALA decode (gfx950): one new token per sequence against a KV cache.
//
// Rule ("MassAlloc Attention: Let Attention Allocate Its Own Compute"; the
// summary page states one tau for training forward, backward, prefill and
// decoding; review page, "One tolerance governs everything" and "Forward:
// online sparse softmax"): the forward rule applied to the block of the G q
// heads that share a KV head, each row seeing L_i = N keys.  Cache tiles of 64
// keys are visited newest first; a tile is kept when some row either has no
// retained mass yet or has exp(tile row max) / retained mass >= tau / N; a
// skipped tile gets no V load and no P.V.
//
// Kernels (tau > 0):
//   mala_dec_score   persistent waves, each streaming a contiguous run of
//                    tiles: S^T = K q^T with 16x16x32 bf16 MFMAs (the G rows
//                    as columns), per-row tile max and shifted sum, and the
//                    shifted exponentials rounded to fp16 as the spill, staged
//                    in LDS and written per run.  Reads every K byte once: the
//                    HBM-bound score discovery.
//   mala_dec_decide  one workgroup per (sequence, KV head): the sequential
//                    rule decided in parallel from an upper and a lower bound
//                    of each tile's retained mass (two workgroup prefix sums),
//                    with an exact serial pass over the tiles the bounds leave
//                    open.
//   mala_dec_pv      persistent workgroups over the kept tiles of all groups:
//                    P = spill x 2^(tile max - lse), V rows of kept tiles only,
//                    fp32 accumulation, one partial per (workgroup, group).
//   mala_dec_sum_combine  sums a group's partials (already normalised) -> bf16 o.
// tau = 0 keeps every tile, so the scan is elided: mala_dec_dense is a fused
// split-K decode (scores, online softmax and P.V per split, eight splits
// merged per workgroup) and mala_dec_dense_combine merges the partials.
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {

namespace {
constexpr int BKD = 64;
constexpr int kScoreWaves = 8;     // waves per score workgroup: all of a CU's waves in one workgroup

// (max, shifted sum) log-sum-exp pairs in base 2: combine is associative.
__device__ __forceinline__ void lse_combine(float& m, float& l, float m2, float l2) {
    const float mn = fmaxf(m, m2);
    if (mn == kNegInf) return;                 // both empty
    l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
    m = mn;
}
}  // namespace

// Keys of sequence b: its cache length, or N without per-sequence lengths; 0
// when the given length lies outside [1, N] (the sequence is then skipped).
__device__ __forceinline__ int dec_len(const DecParams& p, int b) {
    if (!p.seqlens) return p.N;
    const int n = p.seqlens[b];
    return (n >= 1 && n <= p.N) ? n : 0;
}

// Stages one 64-key tile into this wave's LDS slice [64][D] with 16-byte chunk
// c of row r stored at chunk c ^ (r % (D/8)).  Rows past Nb repeat row Nb-1.
template <int D>
__device__ __forceinline__ void stage_k_tile(const DecParams& p, int b, int kh, int t, int Nb, uint16_t* slice) {
    constexpr int QCH = D / 8;
    const int lane = threadIdx.x & 63;
    const uint16_t* kb = p.k + b * p.k_sb + kh * p.k_sh;
#pragma unroll
    for (int n = 0; n < QCH; ++n) {
        const int slot = 64 * n + lane;
        const int r = slot / QCH, pc = slot % QCH;
        const int c = pc ^ (r % QCH);
        int j = t * BKD + r;
        j = j < Nb ? j : Nb - 1;
        load16_to_lds(kb + (int64_t)j * p.k_sl + 8 * c, reinterpret_cast<unsigned char*>(slice) + 1024 * n);
    }
}

// q fragments (B operand: column g = lane%32 for g < G, d = 16 st + 8 hi ..).
template <int D>
__device__ __forceinline__ void load_q_frags(const DecParams& p, int b, int kh, bf16x8* qf) {
    const int lane = threadIdx.x & 63;
    const int g = lane & 31, hi = lane >> 5;
    const bool ok = g < p.G;
    const uint16_t* qrow = p.q + ((int64_t)b * p.Hq + kh * p.G + (ok ? g : 0)) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        const u32x4 x = ok ? *(const u32x4*)(qrow + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
        qf[st] = __builtin_bit_cast(bf16x8, x);
    }
}

// Scores of the staged tile: s[sub][r] is row g = lane%32, key
// 32 sub + 8(r/4) + 4 hi + r%4, base 2, -inf past Nb.
// Scores of the staged tile: s[sub][r] is row g = lane%32, key
// 32 sub + 8(r/4) + 4 hi + r%4, base 2, -inf past Nb.
template <int D>
__device__ __forceinline__ void tile_scores(const DecParams& p, int t, int Nb, const uint16_t* slice,
                                            const bf16x8* qf, f32x16* s) {
    constexpr int QCH = D / 8;
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        const int row = 32 * sub + l32;
        s[sub] = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const int pc = (2 * st + hi) ^ (row % QCH);
            const bf16x8 a = *(const bf16x8*)(slice + row * D + 8 * pc);
            s[sub] = mfma32x32x16(a, qf[st], s[sub]);
        }
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = t * BKD + 32 * sub + 8 * (r >> 2) + 4 * hi + (r & 3);
            s[sub][r] = (j < Nb) ? s[sub][r] * p.scale_log2 : kNegInf;
        }
}

// Score pass.  Persistent waves, eight per workgroup and one workgroup per CU,
// each stream a contiguous run of tiles, the next tile's K fragments in flight
// while the current one is scored.  S^T =
// K q^T with 16x16x32 bf16 MFMAs: the 16 rows of each of the tile's four key
// blocks against the group's q heads as the 16 columns (G <= 16).  Per tile and
// row it yields the base-2 max M and the sum of 2^(s - M); the values
// 2^(s - M) themselves, rounded to fp16, are the spill that the P.V pass reads
// back for kept tiles.  Spill and statistics of a wave's tiles are staged in
// LDS and written when the run ends (or every RUN tiles): small stores
// interleaved with the K stream slow the stream down; written in bursts they
// cost little.
template <int D, int GP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mala_dec_score(const DecParams p) {
    constexpr int KS = D / 32;           // 16x16x32 steps over d
    constexpr int RUN = 8;               // tiles staged per wave before a flush
    __shared__ __attribute__((aligned(16))) uint16_t sSp[kScoreWaves][RUN * GP * BKD];   // [wave][tile][row][key]
    __shared__ float sSt[kScoreWaves][2][GP][RUN];                                       // [wave][max|sum][row][tile]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i16 = lane & 15, q4 = lane >> 4;
    const int G = p.G;
    const int ntask = p.B * p.Hkv * p.nT;
    const int nwave = gridDim.x * kScoreWaves;
    const int per = (ntask + nwave - 1) / nwave;
    // wave-uniform, so the per-tile index arithmetic below runs on the scalar unit
    const int gw = __builtin_amdgcn_readfirstlane(w * gridDim.x + blockIdx.x);   // neighbouring runs on different CUs
    int task = gw * per;
    const int tend = (task + per < ntask) ? task + per : ntask;
    if (task >= tend) return;
    uint16_t* sp = sSp[w];

    // the staged run: group, first tile, tiles staged (consecutive tiles of one group)
    int rgrp = -1, rt0 = 0, rn = 0;
    auto flush = [&]() {
        // this wave's LDS writes have landed before any lane reads them back
        wave_lds_exchange();
        const int nch = rn * G * (BKD / 8);            // 16-byte chunks, contiguous in the tile-major spill
        u32x4* dst = (u32x4*)(p.spill + ((int64_t)rgrp * p.nT + rt0) * G * BKD);
        for (int c = lane; c < nch; c += 64) {
            const int tl = c / (G * 8), rem = c % (G * 8);
            dst[c] = *(const u32x4*)(sp + tl * GP * BKD + rem * 8);
        }
        for (int c = lane; c < rn * G; c += 64) {
            const int g = c / rn, tl = c % rn;
            const int64_t at = ((int64_t)rgrp * G + g) * p.nTp + rt0 + tl;
            p.tmax[at] = sSt[w][0][g][tl];
            p.tsum[at] = sSt[w][1][g][tl];
        }
        wave_lds_exchange();                            // the next run's writes come after these reads
        rn = 0;
    };

    auto load_tile = [&](int tk, bf16x8 (&kf)[4][KS]) {
        const int grp = tk / p.nT, t = tk % p.nT;
        const int b = grp / p.Hkv, kh = grp % p.Hkv;
        const int Nb = dec_len(p, b);
        if (t * BKD >= Nb) return;                     // past this sequence's cache
        const uint16_t* kb = p.k + b * p.k_sb + kh * p.k_sh + 8 * q4;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            int j = t * BKD + 16 * blk + i16;
            j = j < Nb ? j : Nb - 1;                   // rows past Nb are masked below
            const uint16_t* row = kb + (int64_t)j * p.k_sl;
#pragma unroll
            for (int st = 0; st < KS; ++st) kf[blk][st] = *(const bf16x8*)(row + 32 * st);
        }
    };
    int qgrp = -1;
    bf16x8 qf[KS];
    auto score_tile = [&](int tk, const bf16x8 (&kf)[4][KS]) {
        const int grp = tk / p.nT, t = tk % p.nT;
        if (grp != qgrp) {
            // B operand: column i16 = q head of the group, d = 32 st + 8 q4 ..
            const bool ok = i16 < G;
            const uint16_t* qrow = p.q + ((int64_t)(grp / p.Hkv) * p.Hq + (grp % p.Hkv) * G + (ok ? i16 : 0)) * D;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const u32x4 x = ok ? *(const u32x4*)(qrow + 32 * st + 8 * q4) : u32x4{0, 0, 0, 0};
                qf[st] = __builtin_bit_cast(bf16x8, x);
            }
            qgrp = grp;
        }
        // per-call reset owned by this tile
        if (p.bits && lane == 0 && (t % 32) == 0) p.bits[(int64_t)grp * p.nwords + t / 32] = 0u;
        const int Nb = dec_len(p, grp / p.Hkv);
        if (t * BKD >= Nb) return;
        if (rn > 0 && (grp != rgrp || t != rt0 + rn || rn == RUN)) flush();
        if (rn == 0) { rgrp = grp; rt0 = t; }
        const int slot = rn++;
        // C[key][head]: lane i16 + 16 q4 holds head i16, keys 16 blk + 4 q4 + r
        f32x4 c[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            c[blk] = f32x4{};
#pragma unroll
            for (int st = 0; st < KS; ++st) c[blk] = mfma16x16x32(kf[blk][st], qf[st], c[blk]);
        }
        float M = kNegInf;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = t * BKD + 16 * blk + 4 * q4 + r;
                c[blk][r] = (j < Nb) ? c[blk][r] * p.scale_log2 : kNegInf;
                M = fmaxf(M, c[blk][r]);
            }
        M = fmaxf(M, __shfl_xor(M, 16));
        M = wave_max_pair(M);
        float sum = 0.f, e[4][4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                e[blk][r] = fast_exp2(c[blk][r] - M);
                sum += e[blk][r];
            }
        sum += __shfl_xor(sum, 16);
        sum = wave_sum_pair(sum);
        if (i16 < G) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const f16x2v lo = {(_Float16)e[blk][0], (_Float16)e[blk][1]};
                const f16x2v hi = {(_Float16)e[blk][2], (_Float16)e[blk][3]};
                *(u32x2*)(sp + (slot * GP + i16) * BKD + 16 * blk + 4 * q4) =
                    u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            }
            if (q4 == 0) {
                sSt[w][0][i16][slot] = M;
                sSt[w][1][i16][slot] = sum;
            }
        }
    };

    bf16x8 ka[4][KS], kb[4][KS];
    load_tile(task, ka);
    for (; task < tend; task += 2) {
        if (task + 1 < tend) load_tile(task + 1, kb);
        score_tile(task, ka);
        if (task + 1 < tend) {
            if (task + 2 < tend) load_tile(task + 2, ka);
            score_tile(task + 1, kb);
        }
    }
    if (rn > 0) flush();
}

// wave64 prefix sums and reductions built on DPP lane moves: row shifts inside
// 16-lane rows, then row broadcasts of lanes 15 and 31 (lanes whose source is
// out of range add 0).
template <int CTRL, int ROWMASK, bool BOUND0>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, BOUND0));
}
__device__ __forceinline__ float wave_incl_sum(float x) {
    x += dpp_f<0x111, 0xF, true>(x);    // row_shr:1
    x += dpp_f<0x112, 0xF, true>(x);    // row_shr:2
    x += dpp_f<0x114, 0xF, true>(x);    // row_shr:4
    x += dpp_f<0x118, 0xF, true>(x);    // row_shr:8
    x += dpp_f<0x142, 0xA, false>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_f<0x143, 0xC, false>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}
// The value of lane - 1 (0 in lane 0): DPP wave_shr:1.
__device__ __forceinline__ float wave_shr1(float x) { return dpp_f<0x138, 0xF, true>(x); }
// Maximum over the wave (lanes whose source is out of range keep -inf).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_max_step(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(kNegInf), __float_as_int(v), CTRL,
                                                                ROWMASK, 0xF, false)));
}
__device__ __forceinline__ float wave_max_all(float x) {
    x = dpp_max_step<0x111, 0xF>(x);
    x = dpp_max_step<0x112, 0xF>(x);
    x = dpp_max_step<0x114, 0xF>(x);
    x = dpp_max_step<0x118, 0xF>(x);
    x = dpp_max_step<0x142, 0xA>(x);
    x = dpp_max_step<0x143, 0xC>(x);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float readlane_f(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// The sequential decode rule, one wave per (sequence, KV head), 64 tiles per
// chunk (lane = tile, newest first).  State: the retained mass of each row,
// as a reference exponent m and a mass l relative to it (l = 0: nothing
// retained yet, so the next tile is kept).
//
// Each round takes as candidates the active tiles that vote keep under the
// state at the round start (a tile that votes skip under a smaller retained
// mass can never turn to keep, so non-candidates are final), adds to each
// candidate's test the mass of the earlier candidates (an exclusive prefix
// sum), and accepts the candidates up to the first one that then votes skip:
// their prefixes were exact.  That tile is skipped and the next round starts
// after it.
//
// Fast path (linear masses): per chunk the reference is the running maximum
// over every tile seen, a_t = 2^(M_t - ref), x_t = tile sum * a_t, and row g
// votes keep iff a_t >= (tau/N) * (retained + earlier candidates).  Taken when
// no value can leave fp32's normal range (state and tile maxima within 96 of
// the reference, tau/N within 2^+-120); otherwise the chunk runs the same
// rounds with log-sum-exp pairs.
//
// This single-wave form is the general one; mala_dec_decide below runs it
// (on its first wave) for groups outside the linear range.
template <int GP>
__device__ __forceinline__ void decide_one_wave(const DecParams& p, const int Nb) {
    const int grp = blockIdx.x;
    const int lane = threadIdx.x;
    const int G = p.G;
    const int nTb = (Nb + BKD - 1) / BKD;      // this sequence's tiles (p.nT is the stride)
    const float theta = p.log2_tau - (p.seqlens ? (float)log2((double)Nb) : p.log2_N);
    const bool lin_ok = theta >= -120.f && theta <= 120.f;
    const float cthr = fast_exp2(theta);
    float m[GP], l[GP];                   // retained state (identical in all lanes)
#pragma unroll
    for (int g = 0; g < GP; ++g) { m[g] = kNegInf; l[g] = 0.f; }
    int kept = 0;
    int32_t* klist = p.klist + (int64_t)grp * p.nT;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nchunk = (nTb + 63) / 64;
    const float* tmax = p.tmax + (int64_t)grp * G * p.nTp;   // row g at g * nTp
    const float* tsum = p.tsum + (int64_t)grp * G * p.nTp;

    // Group reference: the largest tile max of each row.  When every tile max
    // lies within 96 of it and tau/N within 2^+-120, linear masses relative to
    // it stay inside fp32's normal range for the whole scan, and the rounds run
    // with one fixed reference (no per-chunk reference or rescaling).
    float gref[GP];
    bool linear = lin_ok;
    {
        float mx[GP], mn[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) { mx[g] = kNegInf; mn[g] = __builtin_inff(); }
        // each row is contiguous: 16-byte loads, U of them per row and lane
        // issued together before any is used (the score pass wrote these from
        // other XCDs, so each batch is one far round trip).  The loads are
        // branch-free -- rows past G and indexes past the row re-read valid
        // memory and are discarded -- so none waits for another.
        constexpr int U = GP <= 5 ? 4 : (GP <= 8 ? 2 : 1);
        const int nq = nTb >> 2;
        for (int j0 = 0; j0 < nq; j0 += 64 * U) {
            f32x4 v[U][GP];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + 64 * u + lane;
                const int jc = j < nq ? j : 0;
#pragma unroll
                for (int g = 0; g < GP; ++g)
                    v[u][g] = *(const f32x4*)(tmax + (int64_t)(g < G ? g : 0) * p.nTp + 4 * jc);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = j0 + 64 * u + lane < nq;
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    const float a = fmaxf(fmaxf(v[u][g][0], v[u][g][1]), fmaxf(v[u][g][2], v[u][g][3]));
                    const float b = fminf(fminf(v[u][g][0], v[u][g][1]), fminf(v[u][g][2], v[u][g][3]));
                    mx[g] = ok ? fmaxf(mx[g], a) : mx[g];
                    mn[g] = ok ? fminf(mn[g], b) : mn[g];
                }
            }
        }
        {
            const bool ok = lane < nTb - 4 * nq;
            const int t = ok ? 4 * nq + lane : 0;
            float v[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) v[g] = tmax[(int64_t)(g < G ? g : 0) * p.nTp + t];
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                mx[g] = ok ? fmaxf(mx[g], v[g]) : mx[g];
                mn[g] = ok ? fminf(mn[g], v[g]) : mn[g];
            }
        }
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            gref[g] = (g < G) ? wave_max_all(mx[g]) : 0.f;
            const float lo = (g < G) ? -wave_max_all(-mn[g]) : 0.f;
            linear = linear && (g >= G || lo >= gref[g] - 96.f);
        }
    }

    // accepted tiles of a round: list, bits, count
    auto accept = [&](uint64_t acc, int t) {
        if ((acc >> lane) & 1ull) {
            klist[kept + __builtin_popcountll(acc & lt_mask)] = t;
            if (p.bits) atomicOr(p.bits + (int64_t)grp * p.nwords + t / 32, 1u << (t % 32));
        }
        kept += __builtin_popcountll(acc);
    };

    // Tile statistics stream through an LDS ring of RING chunk slots, DEPTH
    // chunks ahead, with buffer-resource copies (reads before tile 0 return 0;
    // such lanes are invalid anyway).  Slot layout: [max | sum][GP][64]
    // floats, tile t_lo + i of row g at entry 64 g + i.  Every chunk issues GP
    // copies per array (rows past G repeat row 0), which the vmcnt waits count.
    constexpr int DEPTH = (63 / (2 * GP)) < 7 ? ((63 / (2 * GP)) < 1 ? 1 : 63 / (2 * GP)) : 7;
    constexpr int RING = DEPTH + 1;
    __shared__ float sStat[RING][2][64 * GP];
    const __amdgpu_buffer_rsrc_t rmax = make_rsrc(tmax, (uint32_t)(G * p.nTp * 4));
    const __amdgpu_buffer_rsrc_t rsum = make_rsrc(tsum, (uint32_t)(G * p.nTp * 4));
    auto issue_chunk = [&](int c) {
        const int t_lo = nTb - 64 * (c + 1);           // may be negative
        float* dm = sStat[c % RING][0];
        float* ds = sStat[c % RING][1];
#pragma unroll
        for (int i = 0; i < GP; ++i) {
            const int gr = i < G ? i : 0;
            const int t = t_lo + lane;                  // lanes with t < 0 are never used
            const uint32_t off = (t >= 0) ? (uint32_t)((gr * p.nTp + t) * 4) : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rmax, (__attribute__((address_space(3))) void*)(dm + 64 * i), 4,
                                                    (int)off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsum, (__attribute__((address_space(3))) void*)(ds + 64 * i), 4,
                                                    (int)off, 0, 0, 0);
        }
    };
    for (int c = 0; c < DEPTH; ++c)
        if (c < nchunk) issue_chunk(c);
    for (int c = 0; c < nchunk; ++c) {
        const int t = nTb - 1 - (c * 64 + lane);
        const bool valid = t >= 0;
        if (c + DEPTH < nchunk) {
            issue_chunk(c + DEPTH);
            wait_vmcnt<DEPTH * 2 * GP>();
        } else {
            wait_vmcnt<0>();
        }
        float Mg[GP], Sg[GP];
        {
            const float* sm = sStat[c % RING][0];
            const float* ss = sStat[c % RING][1];
            const int i = 63 - lane;                   // t - t_lo
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                Mg[g] = (g < G && valid) ? sm[64 * g + i] : kNegInf;
                Sg[g] = (g < G && valid) ? ss[64 * g + i] : 0.f;
            }
        }
        const bool empty0 = l[0] == 0.f;
        float ref[GP], a[GP], x[GP], Z[GP];
        bool fast;
        if (linear) {
            // the state holds the retained mass relative to gref
            fast = true;
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                const bool row = g < G;
                ref[g] = gref[g];
                a[g] = (row && valid) ? fast_exp2(Mg[g] - gref[g]) : 0.f;
                x[g] = Sg[g] * a[g];
                Z[g] = !row ? 1.f : l[g];
            }
        } else {
            // reference exponents and the range check of the fast path; every
            // loop over rows runs all GP slots branch-free (rows >= G are inert)
            fast = lin_ok;
            bool lane_ok = true;
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                const bool row = g < G;
                ref[g] = row ? fmaxf(m[g], wave_max_all(Mg[g])) : 0.f;
                lane_ok = lane_ok && (!row || !valid || Mg[g] >= ref[g] - 96.f);
                fast = fast && (!row || empty0 || m[g] >= ref[g] - 96.f);
            }
            fast = fast && (__ballot(!lane_ok) == 0ull);
            if (fast) {
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    const bool row = g < G;
                    a[g] = (row && valid) ? fast_exp2(Mg[g] - ref[g]) : 0.f;
                    x[g] = Sg[g] * a[g];
                    Z[g] = !row ? 1.f : (empty0 ? 0.f : l[g] * fast_exp2(m[g] - ref[g]));
                }
            }
        }
        int pos = 0;
        if (fast) {
            bool empty = empty0;
            while (pos < 64) {
                const bool active = valid && lane >= pos;
                bool v0 = empty;
#pragma unroll
                for (int g = 0; g < GP; ++g) v0 = v0 || (a[g] >= cthr * Z[g]);
                v0 = v0 && active;
                const uint64_t K0 = __ballot(v0);
                if (K0 == 0ull) break;                    // the rest of the chunk is skipped
                const int first = __builtin_ctzll(K0);
                float inc[GP], exc[GP];
                bool v1 = empty && lane == first;         // nothing retained before it
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    const float xv = v0 ? x[g] : 0.f;
                    inc[g] = wave_incl_sum(xv);
                    // the previous lane's inclusive sum (inc - xv would cancel
                    // when this tile's mass dwarfs the earlier ones)
                    exc[g] = wave_shr1(inc[g]);
                    v1 = v1 || (a[g] >= cthr * (Z[g] + exc[g]));
                }
                v1 = v1 && v0;
                const uint64_t flips = __ballot(v0 && !v1);
                uint64_t acc;
                int src;
                bool use_exc;
                if (flips == 0ull) {
                    acc = K0; src = 63; use_exc = false;
                } else {
                    const int f = __builtin_ctzll(flips);
                    acc = K0 & ((f == 0) ? 0ull : (~0ull >> (64 - f)));
                    src = f; use_exc = true;
                    pos = f + 1;
                }
                accept(acc, t);
                if (acc) empty = false;
#pragma unroll
                for (int g = 0; g < GP; ++g) Z[g] += readlane_f(use_exc ? exc[g] : inc[g], src);
                if (flips == 0ull) break;
            }
            if (!empty) {
#pragma unroll
                for (int g = 0; g < GP; ++g)
                    if (g < G) {
                        if (!linear) m[g] = ref[g];
                        l[g] = Z[g];
                    }
            }
            continue;
        }
        // ---- log-domain rounds (same structure) for chunks outside the fast range
        float thr[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) thr[g] = (l[g] > 0.f) ? m[g] + fast_log2(l[g]) + theta : kNegInf;
        while (pos < 64) {
            const bool active = valid && lane >= pos;
            bool v0 = false;
#pragma unroll
            for (int g = 0; g < GP; ++g)
                if (g < G) v0 |= (l[g] == 0.f) || (Mg[g] >= thr[g]);
            v0 = v0 && active;
            const uint64_t K0 = __ballot(v0);
            if (K0 == 0ull) break;
            float em[GP], el[GP], im[GP], il[GP];
            bool v1 = false;
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                em[g] = kNegInf; el[g] = 0.f; im[g] = kNegInf; il[g] = 0.f;
                if (g >= G) continue;
                float xm = v0 ? Mg[g] : kNegInf, xl = v0 ? Sg[g] : 0.f;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float ym = __shfl_up(xm, off), yl = __shfl_up(xl, off);
                    if (lane >= off) {
                        float tm = ym, tl = yl;
                        lse_combine(tm, tl, xm, xl);
                        xm = tm; xl = tl;
                    }
                }
                im[g] = xm; il[g] = xl;
                float pm = __shfl_up(xm, 1), pl = __shfl_up(xl, 1);
                if (lane == 0) { pm = kNegInf; pl = 0.f; }
                em[g] = pm; el[g] = pl;
                float zm = m[g], zl = l[g];
                lse_combine(zm, zl, pm, pl);
                v1 |= (zl == 0.f) || (Mg[g] - zm - fast_log2(zl) >= theta);
            }
            v1 = v1 && v0;
            const uint64_t flips = __ballot(v0 && !v1);
            uint64_t acc;
            int src;
            bool use_exc;
            if (flips == 0ull) {
                acc = K0; src = 63; use_exc = false;
            } else {
                const int f = __builtin_ctzll(flips);
                acc = K0 & ((f == 0) ? 0ull : (~0ull >> (64 - f)));
                src = f; use_exc = true;
                pos = f + 1;
            }
            accept(acc, t);
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                if (g >= G) continue;
                const float nm = readlane_f(use_exc ? em[g] : im[g], src);
                const float nl = readlane_f(use_exc ? el[g] : il[g], src);
                lse_combine(m[g], l[g], nm, nl);
                thr[g] = (l[g] > 0.f) ? m[g] + fast_log2(l[g]) + theta : kNegInf;
            }
            if (flips == 0ull) break;
        }
    }
    if (lane == 0) {
        p.kcount[grp] = kept;
        if (p.kept_tiles) p.kept_tiles[grp] = kept;
    }
    if (linear) {
#pragma unroll
        for (int g = 0; g < GP; ++g)
            if (g < G) m[g] = gref[g];
    }
    if (lane < G) {
        float mm = kNegInf, ll = 0.f;
#pragma unroll
        for (int g = 0; g < GP; ++g)
            if (g == lane) { mm = m[g]; ll = l[g]; }
        const float lz2 = mm + fast_log2(ll);
        p.lse2[(int64_t)grp * G + lane] = lz2;
        const int b = grp / p.Hkv, kh = grp % p.Hkv;
        p.lse[(int64_t)b * p.Hq + kh * G + lane] = lz2 * kLn2;
    }
}

// Exclusive prefix sums over the workgroup of N values per thread (thread
// order is the order of the sums) and their totals.  sW holds one entry per
// wave and value; the workgroup must not be using it.
template <int N, int NW>
__device__ __forceinline__ void block_excl_scan(float (&v)[N], float (&tot)[N], float (*sW)[N]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    float inc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) inc[i] = wave_incl_sum(v[i]);
    if (lane == 63)
#pragma unroll
        for (int i = 0; i < N; ++i) sW[w][i] = inc[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float off = 0.f, all = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            const float s = sW[w2][i];
            off += (w2 < w) ? s : 0.f;
            all += s;
        }
        // the previous lane's inclusive sum, never inc minus this lane's value
        v[i] = off + wave_shr1(inc[i]);
        tot[i] = all;
    }
    __syncthreads();
}

// The sequential decode rule for one (sequence, KV head), decided in parallel
// with bounds.  Visit position v = 0, 1, .. is tile nTb-1-v (newest first); Z
// is each row's retained mass, a_v = 2^(M_v - ref) and x_v = tile sum * a_v
// per row, linear masses against the row's largest tile max.  The rule keeps
// tile v iff some row has Z(v) = 0 or a_v >= (tau/N) Z(v), Z(v) the mass of
// the kept tiles before v.  Z(v) is at most the mass of ALL earlier tiles
// (upper bound U) and at least the mass of the earlier tiles already known to
// be kept (lower bound R).  So a tile that passes against U is surely kept,
// one that fails against R is surely skipped, both from two prefix sums over
// the workgroup, and only the rest -- ambiguous tiles, rare because skipped
// tiles carry little mass -- need the sequential rule: a serial pass over
// them in visit order with Z(v) = R(v) + the mass of the ambiguous tiles it
// keeps before v.  The decisions are those of the sequential rule exactly.
//
// Tiles are taken in chunks of CH positions (the state carried across);
// rows whose tile maxima span more than 2^96, or tau/N beyond 2^+-120, leave
// fp32's range for linear masses: such groups run the round-based
// log-sum-exp form decide_one_wave on the first wave.
template <int GP>
constexpr int decide_tpt() { return GP <= 5 ? 4 : (GP <= 8 ? 2 : 1); }

template <int GP>
__global__ __launch_bounds__(512) void mala_dec_decide(const DecParams p) {
    constexpr int NTH = 512, NW = NTH / 64;
    constexpr int TPT = decide_tpt<GP>();
    constexpr int CH = NTH * TPT;
    constexpr int AMBCAP = 256;            // ambiguous tiles resolved per serial pass
    __shared__ float sW[NW][GP + 2];
    __shared__ float sRef[NW][GP][2];
    __shared__ float sAmb[AMBCAP][3][GP];   // a, x, R of each ambiguous tile of the pass
    __shared__ int sAmbKeep[AMBCAP];
    __shared__ float sE[GP];
    const int grp = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = p.G;
    const int Nb = dec_len(p, grp / p.Hkv);
    if (Nb == 0) {                              // skipped sequence: nothing retained
        if (tid == 0) {
            p.kcount[grp] = 0;
            if (p.kept_tiles) p.kept_tiles[grp] = 0;
        }
        return;
    }
    const int nTb = (Nb + BKD - 1) / BKD;      // this sequence's tiles (p.nT is the stride)
    const float theta = p.log2_tau - (p.seqlens ? (float)log2((double)Nb) : p.log2_N);
    const bool lin_ok = theta >= -120.f && theta <= 120.f;
    const float cthr = fast_exp2(theta);
    const float* tmax = p.tmax + (int64_t)grp * G * p.nTp;   // row g at g * nTp
    const float* tsum = p.tsum + (int64_t)grp * G * p.nTp;

    const int nchunk = (nTb + CH - 1) / CH;
    // This thread's positions of chunk c: v = c CH + TPT tid + j, tile nTb - 1 - v
    // (TPT consecutive tiles, one 16-byte load per row when they are aligned).
    float M[TPT][GP], S[TPT][GP];
    bool valid[TPT];
    int tile[TPT];
    auto load_chunk = [&](int c) {
        const int top = nTb - 1 - (c * CH + TPT * tid);          // tile of j = 0
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            tile[j] = top - j;
            valid[j] = tile[j] >= 0;
        }
        if (TPT == 4 && (top - 3) >= 0 && ((top - 3) & 3) == 0) {
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                const int64_t at = (int64_t)(g < G ? g : 0) * p.nTp + (top - 3);
                const f32x4 m4 = *(const f32x4*)(tmax + at);
                const f32x4 s4 = *(const f32x4*)(tsum + at);
#pragma unroll
                for (int j = 0; j < TPT; ++j) { M[j][g] = m4[3 - j]; S[j][g] = s4[3 - j]; }
            }
        } else {
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const int t = valid[j] ? tile[j] : 0;
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    const int64_t at = (int64_t)(g < G ? g : 0) * p.nTp + t;
                    M[j][g] = tmax[at];
                    S[j][g] = tsum[at];
                }
            }
        }
    };
    load_chunk(0);

    // Row references: the largest tile max, and whether the smallest lies within 96 of it.
    float gref[GP];
    bool linear = lin_ok;
    {
        float mx[GP], mn[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) { mx[g] = kNegInf; mn[g] = __builtin_inff(); }
        if (nchunk == 1) {                     // every tile is in this thread's registers already
#pragma unroll
            for (int j = 0; j < TPT; ++j)
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    mx[g] = valid[j] ? fmaxf(mx[g], M[j][g]) : mx[g];
                    mn[g] = valid[j] ? fminf(mn[g], M[j][g]) : mn[g];
                }
        } else
        for (int t0 = tid; t0 < nTb; t0 += TPT * NTH) {
            float v[TPT][GP];
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const int t = t0 + j * NTH;
#pragma unroll
                for (int g = 0; g < GP; ++g) v[j][g] = tmax[(int64_t)(g < G ? g : 0) * p.nTp + (t < nTb ? t : 0)];
            }
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const bool ok = t0 + j * NTH < nTb;
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    mx[g] = ok ? fmaxf(mx[g], v[j][g]) : mx[g];
                    mn[g] = ok ? fminf(mn[g], v[j][g]) : mn[g];
                }
            }
        }
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float a = wave_max_all(mx[g]);
            const float b = -wave_max_all(-mn[g]);
            if (lane == 0) { sRef[w][g][0] = a; sRef[w][g][1] = b; }
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            float a = kNegInf, b = __builtin_inff();
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) { a = fmaxf(a, sRef[w2][g][0]); b = fminf(b, sRef[w2][g][1]); }
            gref[g] = (g < G) ? a : 0.f;
            linear = linear && (g >= G || b >= a - 96.f);
        }
    }
    if (!linear) {
        if (w == 0) decide_one_wave<GP>(p, Nb);
        return;
    }

    int32_t* klist = p.klist + (int64_t)grp * p.nT;
    float Z[GP];                                // retained mass so far (identical in every thread)
#pragma unroll
    for (int g = 0; g < GP; ++g) Z[g] = 0.f;
    int kbase = 0;
    for (int c = 0; c < nchunk; ++c) {
        float a[TPT][GP], x[TPT][GP];
        {
            if (c > 0) load_chunk(c);
#pragma unroll
            for (int j = 0; j < TPT; ++j)
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    const bool ok = valid[j] && g < G;
                    a[j][g] = ok ? fast_exp2(M[j][g] - gref[g]) : 0.f;
                    x[j][g] = ok ? S[j][g] * a[j][g] : 0.f;
                }
        }
        // upper bound: the mass of every earlier tile
        bool sk[TPT];
        {
            float pre[GP], tot[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                pre[g] = 0.f;
#pragma unroll
                for (int j = 0; j < TPT; ++j) pre[g] += x[j][g];
            }
            block_excl_scan<GP, NW>(pre, tot, (float(*)[GP])sW);
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                bool k = false;
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    k = k || (g < G && a[j][g] >= cthr * (Z[g] + pre[g]));
                    pre[g] += x[j][g];
                }
                sk[j] = valid[j] && k;
            }
        }
        // lower bound: the mass of the earlier surely-kept tiles (scanned with
        // their count, which places the kept tiles when none is ambiguous)
        bool amb[TPT];
        float R[TPT][GP];
        float sktot[GP];
        int nk_before, nk_total, na = 0;
        {
            float pre[GP + 1], tot[GP + 1];
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                pre[g] = 0.f;
#pragma unroll
                for (int j = 0; j < TPT; ++j) pre[g] += sk[j] ? x[j][g] : 0.f;
            }
            pre[GP] = 0.f;
#pragma unroll
            for (int j = 0; j < TPT; ++j) pre[GP] += sk[j] ? 1.f : 0.f;
            block_excl_scan<GP + 1, NW>(pre, tot, (float(*)[GP + 1])sW);
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                bool k = false;
#pragma unroll
                for (int g = 0; g < GP; ++g) {
                    R[j][g] = Z[g] + pre[g];
                    k = k || (g < G && a[j][g] >= cthr * R[j][g]);
                    pre[g] += sk[j] ? x[j][g] : 0.f;
                }
                amb[j] = valid[j] && !sk[j] && k;
                na += amb[j] ? 1 : 0;
            }
#pragma unroll
            for (int g = 0; g < GP; ++g) sktot[g] = tot[g];
            nk_before = (int)pre[GP];
            nk_total = (int)tot[GP];
        }
        bool keep[TPT];
#pragma unroll
        for (int j = 0; j < TPT; ++j) keep[j] = sk[j];
        float Etot[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) Etot[g] = 0.f;
        if (__syncthreads_or(na)) {
            // the sequential rule over the ambiguous tiles, in visit order,
            // AMBCAP at a time; E = mass of the ambiguous tiles kept so far
            float pa[1] = {(float)na}, ta[1];
            block_excl_scan<1, NW>(pa, ta, (float(*)[1])sW);
            const int namb_before = (int)pa[0], namb_total = (int)ta[0];
            if (tid == 0)
#pragma unroll
                for (int g = 0; g < GP; ++g) sE[g] = 0.f;
            for (int r0 = 0; r0 < namb_total; r0 += AMBCAP) {
                int idx = namb_before;
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    if (amb[j]) {
                        if (idx >= r0 && idx < r0 + AMBCAP)
#pragma unroll
                            for (int g = 0; g < GP; ++g) {
                                sAmb[idx - r0][0][g] = a[j][g];
                                sAmb[idx - r0][1][g] = x[j][g];
                                sAmb[idx - r0][2][g] = R[j][g];
                            }
                        ++idx;
                    }
                }
                __syncthreads();
                if (tid == 0) {
                    float E[GP];
#pragma unroll
                    for (int g = 0; g < GP; ++g) E[g] = sE[g];
                    const int n = (namb_total - r0 < AMBCAP) ? namb_total - r0 : AMBCAP;
                    for (int i = 0; i < n; ++i) {
                        bool k = false;
#pragma unroll
                        for (int g = 0; g < GP; ++g) k = k || (g < G && sAmb[i][0][g] >= cthr * (sAmb[i][2][g] + E[g]));
                        if (k)
#pragma unroll
                            for (int g = 0; g < GP; ++g) E[g] += sAmb[i][1][g];
                        sAmbKeep[i] = k ? 1 : 0;
                    }
#pragma unroll
                    for (int g = 0; g < GP; ++g) sE[g] = E[g];
                }
                __syncthreads();
                idx = namb_before;
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    if (amb[j]) {
                        if (idx >= r0 && idx < r0 + AMBCAP) keep[j] = sAmbKeep[idx - r0] != 0;
                        ++idx;
                    }
                }
                __syncthreads();
            }
#pragma unroll
            for (int g = 0; g < GP; ++g) Etot[g] = sE[g];
            // kept tiles before each position, ambiguous ones included
            float pk[1] = {0.f}, tk[1];
#pragma unroll
            for (int j = 0; j < TPT; ++j) pk[0] += keep[j] ? 1.f : 0.f;
            block_excl_scan<1, NW>(pk, tk, (float(*)[1])sW);
            nk_before = (int)pk[0];
            nk_total = (int)tk[0];
        }
        // the kept tiles, newest first
        {
            int o = kbase + nk_before;
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                if (keep[j]) {
                    klist[o++] = tile[j];
                    if (p.bits) atomicOr(p.bits + (int64_t)grp * p.nwords + tile[j] / 32, 1u << (tile[j] % 32));
                }
            }
        }
        kbase += nk_total;
#pragma unroll
        for (int g = 0; g < GP; ++g) Z[g] += sktot[g] + Etot[g];
    }
    if (tid == 0) {
        p.kcount[grp] = kbase;
        if (p.kept_tiles) p.kept_tiles[grp] = kbase;
    }
    if (tid < G) {
        float zz = 0.f, rr = 0.f;
#pragma unroll
        for (int g = 0; g < GP; ++g)
            if (g == tid) { zz = Z[g]; rr = gref[g]; }
        const float lz2 = rr + fast_log2(zz);
        p.lse2[(int64_t)grp * G + tid] = lz2;
        const int b = grp / p.Hkv, kh = grp % p.Hkv;
        p.lse[(int64_t)b * p.Hq + kh * G + tid] = lz2 * kLn2;
    }
}

// Integer wave prefix sums (DPP, as wave_incl_sum) and a workgroup scan of one
// int per thread (thread order), with the total.
template <int CTRL, int ROWMASK, bool BOUND0>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, BOUND0);
}
__device__ __forceinline__ int wave_incl_sum_i(int x) {
    x += dpp_i<0x111, 0xF, true>(x);
    x += dpp_i<0x112, 0xF, true>(x);
    x += dpp_i<0x114, 0xF, true>(x);
    x += dpp_i<0x118, 0xF, true>(x);
    x += dpp_i<0x142, 0xA, false>(x);
    x += dpp_i<0x143, 0xC, false>(x);
    return x;
}
template <int NW>
__device__ __forceinline__ int block_excl_scan_i(int v, int& tot, int* sWi) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int inc = wave_incl_sum_i(v);
    if (lane == 63) sWi[w] = inc;
    __syncthreads();
    int off = 0, all = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
        const int s = sWi[w2];
        off += (w2 < w) ? s : 0;
        all += s;
    }
    __syncthreads();
    tot = all;
    return off + inc - v;
}

// P.V over the kept tiles of every group.  The kept lists of all groups,
// concatenated in group order, are cut into equal ranges, one per workgroup,
// so no workgroup waits on an empty list and none carries a group's whole
// load; its four waves take every fourth tile of each group's part of the
// range.  For a tile, O^T += V^T P^T runs on 16x16x32 bf16 MFMAs: d in 16-row
// blocks, the group's q heads as the 16 columns, keys as the contraction.
// P = (spilled fp16 2^(s - M)) x 2^(M - lse), M the row's tile max: the fp16
// part is split exactly into two bf16 parts (high: the value rounded to bf16,
// low: the rest, which fits bf16 exactly), each taken by its own MFMA, so the
// product with bf16 V is that of fp16 P in fp32 arithmetic; the factor
// 2^(M - lse) scales the tile's contribution per column afterwards.  V^T
// operands come from the tile staged in LDS (global -> LDS copies, 16-byte
// chunks XOR-swizzled by row) through transposing reads.  For each group its
// range meets, a workgroup writes one partial output (already normalised) to
// slot workgroup + group: a workgroup meets groups in increasing order, so no
// two (workgroup, group) pairs share a slot.  The workgroup that holds a
// group's first kept tile records the group's first slot and slot count
// (pvinfo).
template <int D, int GP>
__global__ __launch_bounds__(256) void mala_dec_pv(const DecParams p) {
    constexpr int NB = D / 16;           // 16-row blocks of d
    constexpr int CH = D / 8;            // 16-byte chunks per V row
    constexpr int RPC = 64 / CH;         // V rows per 1 KB global -> LDS copy
    constexpr int TLCAP = 1024;          // tile indices staged per pass
    __shared__ __attribute__((aligned(16))) uint16_t sV[4][BKD * D];   // one V tile per wave
    __shared__ int sTl[TLCAP];
    __shared__ int sWi[4];
    __shared__ int sFound[2];
    __shared__ int sKc[256];
    float (*sRed)[16][D] = reinterpret_cast<float (*)[16][D]>(&sV[0][0]);   // [wave][head][d], after the tiles
    static_assert(sizeof(sV) >= 4 * 16 * D * sizeof(float), "reduction buffer");
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int j16 = lane & 15, q4 = lane >> 4;
    const int G = p.G;
    const int ngrp = p.B * p.Hkv;
    const int wg = blockIdx.x;

    // total kept tiles T, this workgroup's range [s, e), and the group holding
    // item s with its first item.  Up to 256 groups one scan gives all of it
    // (thread g holds group g's count and prefix), and the counts stay in LDS.
    int T = 0, per = 0, s = 0, e = 0;
    if (ngrp <= 256) {
        const int kc = tid < ngrp ? p.kcount[tid] : 0;
        sKc[tid] = kc;
        int tot;
        const int pre = block_excl_scan_i<4>(kc, tot, sWi);
        T = tot;
        if (T == 0) return;
        per = (T + gridDim.x - 1) / gridDim.x;
        s = wg * per;
        e = (s + per < T) ? s + per : T;
        if (s >= e) return;
        if (tid < ngrp && pre <= s && s < pre + kc) { sFound[0] = tid; sFound[1] = pre; }
        __syncthreads();
    } else {
        int c = 0;
        for (int g = tid; g < ngrp; g += 256) c += p.kcount[g];
        int tot;
        block_excl_scan_i<4>(c, tot, sWi);
        T = tot;
        if (T == 0) return;
        per = (T + gridDim.x - 1) / gridDim.x;
        s = wg * per;
        e = (s + per < T) ? s + per : T;
        if (s >= e) return;
        int carry = 0;
        for (int g0 = 0; g0 < ngrp; g0 += 256) {
            const int g = g0 + tid;
            const int kc = g < ngrp ? p.kcount[g] : 0;
            const int pre = carry + block_excl_scan_i<4>(kc, tot, sWi);
            if (g < ngrp && pre <= s && s < pre + kc) { sFound[0] = g; sFound[1] = pre; }
            carry += tot;
            if (carry > s) break;                       // uniform: every thread holds the same carry
        }
        __syncthreads();
    }
    auto kcount_of = [&](int g) { return ngrp <= 256 ? sKc[g] : p.kcount[g]; };
    int g = sFound[0];
    int pre = sFound[1];
    uint16_t* vt = sV[w];
    int i = s;
    while (i < e) {                                     // uniform over the workgroup
        const int kc = kcount_of(g);
        const int seg_end = (pre + kc < e) ? pre + kc : e;
        if (seg_end > i) {
            const int b = g / p.Hkv, kh = g % p.Hkv;
            const int Nb = dec_len(p, b);
            const int n = seg_end - i;
            const int32_t* kl = p.klist + (int64_t)g * p.nT + (i - pre);
            const uint16_t* vbase = p.v + b * p.v_sb + kh * p.v_sh;
            // column (q head) of this lane in the B operand and the output
            const bool hv = j16 < G;
            const int hh = hv ? j16 : 0;
            const float lse_h = p.lse2[(int64_t)g * G + hh];
            f32x4 acc[NB];
#pragma unroll
            for (int m = 0; m < NB; ++m) acc[m] = f32x4{};
            for (int m0 = 0; m0 < n; m0 += TLCAP) {
                const int nb = (n - m0 < TLCAP) ? n - m0 : TLCAP;
                for (int m = tid; m < nb; m += 256) sTl[m] = kl[m0 + m];
                __syncthreads();
                for (int m = w; m < nb; m += 4) {
                    const int t = sTl[m];
                    // V tile -> this wave's LDS slice, 1 KB (RPC rows) per copy: lane l lands
                    // at row RPC k + l / CH, position l % CH, and holds global chunk
                    // (l % CH) ^ (row % 8)
#pragma unroll
                    for (int k = 0; k < BKD / RPC; ++k) {
                        const int row = RPC * k + lane / CH;
                        int key = t * BKD + row;
                        key = key < Nb ? key : Nb - 1;
                        const int ch = ((lane % CH) ^ (row & 7)) & (CH - 1);
                        load16_to_lds(vbase + (int64_t)key * p.v_sl + 8 * ch, vt + k * RPC * D);
                    }
                    // P of the tile for head j16, keys 32 st + 8 q4 .. +7, and its factor
                    const uint16_t* sp = p.spill + (((int64_t)g * p.nT + t) * G + hh) * BKD + 8 * q4;
                    const u32x4 p0 = *(const u32x4*)(sp);
                    const u32x4 p1 = *(const u32x4*)(sp + 32);
                    const float tm = p.tmax[((int64_t)g * G + hh) * p.nTp + t];
                    const float f = hv ? fast_exp2(tm - lse_h) : 0.f;
                    // exact split of the fp16 values into bf16 high and low parts
                    bf16x8 bh[2], bl[2];
                    {
                        const uint32_t ph[2][4] = {{p0[0], p0[1], p0[2], p0[3]}, {p1[0], p1[1], p1[2], p1[3]}};
#pragma unroll
                        for (int st = 0; st < 2; ++st)
#pragma unroll
                            for (int h = 0; h < 4; ++h) {
                                const float a0 = f16_lo_to_float(ph[st][h]), a1 = f16_hi_to_float(ph[st][h]);
                                const __bf16 h0 = to_bf16(a0), h1 = to_bf16(a1);
                                bh[st][2 * h] = h0;
                                bh[st][2 * h + 1] = h1;
                                bl[st][2 * h] = to_bf16(a0 - (float)h0);
                                bl[st][2 * h + 1] = to_bf16(a1 - (float)h1);
                            }
                    }
                    // the copies above are the only writes to vt; every lane's part has landed
                    __builtin_amdgcn_s_waitcnt(0);
                    wave_lds_exchange();
#pragma unroll
                    for (int mb = 0; mb < NB; ++mb) {
                        f32x4 c = f32x4{};
#pragma unroll
                        for (int st = 0; st < 2; ++st) {
                            // A[i][k] = V[32 st + k][16 mb + i]: lane j16 + 16 q4 reads keys 32 st + 8 q4 ..
                            // +3 and +4 .. +7 of column 16 mb + j16 (transposing reads: lane x of
                            // the 16-lane group addresses key r0 + x/4, columns 16 mb + 4 (x%4) ..)
                            bf16x8 a;
#pragma unroll
                            for (int hlf = 0; hlf < 2; ++hlf) {
                                const int r = 32 * st + 8 * q4 + 4 * hlf + (j16 >> 2);
                                const int col = 16 * mb + 4 * (j16 & 3);
                                const int pos = ((col >> 3) ^ (r & 7)) & (CH - 1);
                                const u32x2 x = lds_read_tr16(vt + r * D + pos * 8 + (col & 7));
                                const bf16x8 xx = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], 0u, 0u});
#pragma unroll
                                for (int u = 0; u < 4; ++u) a[4 * hlf + u] = xx[u];
                            }
                            c = mfma16x16x32(a, bh[st], c);
                            c = mfma16x16x32(a, bl[st], c);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mb][r] += f * c[r];
                    }
                    wave_lds_exchange();               // the next tile's copies come after these reads
                }
                __syncthreads();                          // sTl is rewritten by the next pass
            }
            // acc[mb][r] = O^T[16 mb + 4 q4 + r][head j16] of this wave's tiles; sum the waves
#pragma unroll
            for (int mb = 0; mb < NB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) sRed[w][j16][16 * mb + 4 * q4 + r] = acc[mb][r];
            __syncthreads();
            float* po = p.part_o + ((int64_t)(wg + g) * G) * D;
            for (int x = tid; x < G * D; x += 256) {
                const int h = x / D, d = x % D;
                po[x] = sRed[0][h][d] + sRed[1][h][d] + sRed[2][h][d] + sRed[3][h][d];
            }
            if (i == pre && tid == 0) {
                p.pvinfo[2 * g] = wg;                                      // first slot's workgroup
                p.pvinfo[2 * g + 1] = (pre + kc - 1) / per - wg + 1;        // slots
            }
            __syncthreads();                              // sRed (the V slices) is rewritten next
            i = seg_end;
        }
        pre += kc;
        ++g;
    }
}

// Sum of the P.V partials of a group (already normalised by the final LSE) ->
// bf16 o.  One workgroup per (group, row, 32-wide d slice): 8 slot classes x
// 32 d, the slots of each class summed in order.
template <int D>
__global__ __launch_bounds__(256) void mala_dec_sum_combine(const DecParams p) {
    __shared__ float sO[8][32];
    const int tid = threadIdx.x;
    const int grp = blockIdx.x, g = blockIdx.y, dq = blockIdx.z;
    const int G = p.G;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    if (dec_len(p, b) == 0) return;              // skipped sequence: o is left as it was
    const int wg0 = p.pvinfo[2 * grp], ns = p.pvinfo[2 * grp + 1];
    const int d = 32 * dq + (tid & 31), cls = tid >> 5;
    float osum = 0.f;
#pragma unroll 4
    for (int s = cls; s < ns; s += 8) osum += p.part_o[((int64_t)(wg0 + s + grp) * G + g) * D + d];
    sO[cls][tid & 31] = osum;
    __syncthreads();
    if (tid < 32) {
        float o = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o += sO[c][tid];
        p.o[((int64_t)b * p.Hq + kh * G + g) * D + 32 * dq + tid] = (uint16_t)float_to_bf16_bits(o);
    }
}

// tau = 0: fused split-K decode.  Wave (group, split) streams the split's
// tiles: K fragments in registers one tile ahead, the V tile staged in the
// wave's LDS slice, S^T = K q^T and the online softmax per q head, then
// O^T += V^T P^T on 16x16x32 bf16 MFMAs.  The contraction takes the keys in a
// permuted order -- position 8 q4 + u of step st is key 32 st + 4 q4 + u and
// position 8 q4 + 4 + u is key 32 st + 16 + 4 q4 + u -- so a lane's B
// operand is exactly the eight probabilities its score registers hold, and
// the transposing V reads take the same order.  P (fp32) is split into a bf16
// high part and a bf16 low part (the rest, rounded), each taken by its own
// MFMA: about 16 significant bits of P.  Eight waves per workgroup (one
// workgroup per CU) take eight consecutive splits of one group; the
// workgroup merges their (max, sum, output) through LDS and writes one
// partial, and mala_dec_dense_combine merges a group's partials.
template <int D, int GP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mala_dec_dense(const DecParams p) {
    constexpr int KS = D / 32;           // 16x16x32 steps over d
    constexpr int NB = D / 16;           // 16-row blocks of d
    constexpr int CH = D / 8;            // 16-byte chunks per V row
    constexpr int RPC = 64 / CH;         // V rows per 1 KB copy
    constexpr int NWV = 8;
    constexpr int NKL = 4 * KS;          // K load instructions per tile
    __shared__ __attribute__((aligned(16))) uint16_t sV[NWV][BKD * D];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[NWV][KS * 64 * 8];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int i16 = lane & 15, q4 = lane >> 4;
    const int G = p.G;
    // The eight waves of a workgroup take eight consecutive splits of one group
    // (the number of splits per group is a multiple of 8).
    const int gw = __builtin_amdgcn_readfirstlane((int)blockIdx.x * NWV + w);
    const int grp = gw / p.nsplit, s = gw % p.nsplit;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    const int Nb = dec_len(p, b);
    const int nTb = (Nb + BKD - 1) / BKD;
    const int t0 = s * p.tiles_per_split;
    const int t1 = (t0 + p.tiles_per_split < nTb) ? t0 + p.tiles_per_split : nTb;   // may be empty
    const uint16_t* kbase = p.k + b * p.k_sb + kh * p.k_sh + 8 * q4;
    const uint16_t* vbase = p.v + b * p.v_sb + kh * p.v_sh;
    uint16_t* vt = sV[w];
    // B operand of the scores, kept in this wave's LDS slice (registers go to
    // the K tiles): column i16 = q head of the group, d = 32 st + 8 q4 ..
    // Loaded first and written to LDS once the first K tile's loads are out,
    // so the kernel's first cache reads do not wait for it.
    u32x4 qx[KS];
    {
        const bool ok = i16 < G;
        const uint16_t* qrow = p.q + ((int64_t)b * p.Hq + kh * G + (ok ? i16 : 0)) * D;
#pragma unroll
        for (int st = 0; st < KS; ++st) qx[st] = ok ? *(const u32x4*)(qrow + 32 * st + 8 * q4) : u32x4{0, 0, 0, 0};
    }
    auto stage_q = [&]() {
#pragma unroll
        for (int st = 0; st < KS; ++st) *(u32x4*)(&sQ[w][(st * 64 + lane) * 8]) = qx[st];
        wave_lds_exchange();
    };
    auto qfrag = [&](int st) -> bf16x8 { return *(const bf16x8*)(&sQ[w][(st * 64 + lane) * 8]); };
    // A operand of the scores: row 16 blk + i16 of the tile, d = 32 st + 8 q4 ..
    auto load_k = [&](int t, bf16x8 (&kf)[4][KS]) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            int j = t * BKD + 16 * blk + i16;
            j = j < Nb ? j : Nb - 1;                   // rows past Nb are masked
            const uint16_t* row = kbase + (int64_t)j * p.k_sl;
#pragma unroll
            for (int st = 0; st < KS; ++st) kf[blk][st] = *(const bf16x8*)(row + 32 * st);
        }
    };
    // V tile -> this wave's LDS slice, 1 KB (RPC rows) per copy: lane l lands at
    // row RPC k + l / CH, position l % CH, and holds chunk (l % CH) ^ (row % 8)
    auto stage_v = [&](int t) {
#pragma unroll
        for (int k = 0; k < BKD / RPC; ++k) {
            const int row = RPC * k + lane / CH;
            int key = t * BKD + row;
            key = key < Nb ? key : Nb - 1;
            const int ch = ((lane % CH) ^ (row & 7)) & (CH - 1);
            global16_to_lds_asm(vbase + (int64_t)key * p.v_sl + 8 * ch, vt + k * RPC * D);
        }
    };
    float m_run = kNegInf, l_run = 0.f;           // of head i16 (identical in its four lanes)
    f32x4 acc[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m) acc[m] = f32x4{};

    // One tile: V(t) is in flight (issued before the next K tile's loads).
    auto tile = [&](int t, const bf16x8 (&kf)[4][KS], bool more) {
        f32x4 c[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            c[blk] = f32x4{};
#pragma unroll
            for (int st = 0; st < KS; ++st) c[blk] = mfma16x16x32(kf[blk][st], qfrag(st), c[blk]);
        }
        // c[blk][r]: head i16, key 16 blk + 4 q4 + r
        float M = kNegInf;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = t * BKD + 16 * blk + 4 * q4 + r;
                c[blk][r] = (j < Nb) ? c[blk][r] * p.scale_log2 : kNegInf;
                M = fmaxf(M, c[blk][r]);
            }
        M = fmaxf(M, __shfl_xor(M, 16));
        M = wave_max_pair(M);
        const float mn = fmaxf(m_run, M);             // finite: the tile holds a key below Nb
        const float alpha = fast_exp2(m_run - mn);    // 0 for the first tile
        float sum = 0.f;
        bf16x8 bh[2], bl[2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float pv = fast_exp2(c[2 * st + hf][u] - mn);
                    sum += pv;
                    const __bf16 h = to_bf16(pv);
                    bh[st][4 * hf + u] = h;
                    bl[st][4 * hf + u] = to_bf16(pv - (float)h);
                }
        sum += __shfl_xor(sum, 16);
        sum = wave_sum_pair(sum);
        l_run = l_run * alpha + sum;
        m_run = mn;
        if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][r] *= alpha;
        }
        // V(t) has landed once at most the next tile's K loads are outstanding
        if (more) wait_vmcnt<NKL>();
        else wait_vmcnt<0>();
        wave_lds_exchange();
#pragma unroll
        for (int mb = 0; mb < NB; ++mb) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                // A[i][k] = V[key of position k][16 mb + i]: rows 32 st + 16 hlf + 4 q4 .. +3
                bf16x8 a;
#pragma unroll
                for (int hlf = 0; hlf < 2; ++hlf) {
                    const int r = 32 * st + 16 * hlf + 4 * q4 + (i16 >> 2);
                    const int col = 16 * mb + 4 * (i16 & 3);
                    const int pos = ((col >> 3) ^ (r & 7)) & (CH - 1);
                    const u32x2 x = lds_read_tr16(vt + r * D + pos * 8 + (col & 7));
                    const bf16x8 xx = __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], 0u, 0u});
#pragma unroll
                    for (int u = 0; u < 4; ++u) a[4 * hlf + u] = xx[u];
                }
                acc[mb] = mfma16x16x32(a, bh[st], acc[mb]);
                acc[mb] = mfma16x16x32(a, bl[st], acc[mb]);
            }
        }
        wave_lds_exchange();                          // the next tile's copies come after these reads
    };

    if (t0 < t1) {
        bf16x8 ka[4][KS], kb[4][KS];
        load_k(t0, ka);
        stage_q();
        for (int t = t0; t < t1; t += 2) {
            stage_v(t);
            const bool m1 = t + 1 < t1;
            if (m1) load_k(t + 1, kb);
            tile(t, ka, m1);
            if (!m1) break;
            stage_v(t + 1);
            const bool m2 = t + 2 < t1;
            if (m2) load_k(t + 2, ka);
            tile(t + 1, kb, m2);
        }
    }
    // The workgroup's partial: the eight splits merged (log-sum-exp) through LDS,
    // then (max, sum) per head and the unnormalised output of partial s / 8.
    __syncthreads();                                  // every wave is done with its V slice
    float (*sRed)[GP][D] = reinterpret_cast<float (*)[GP][D]>(&sV[0][0]);            // [wave][head][d]
    float (*sML)[GP][2] = reinterpret_cast<float (*)[GP][2]>(&sRed[NWV][0][0]);        // [wave][head][max|sum]
    static_assert(sizeof(sV) >= NWV * GP * (D + 2) * sizeof(float), "reduction buffer");
    if (i16 < GP) {
#pragma unroll
        for (int mb = 0; mb < NB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sRed[w][i16][16 * mb + 4 * q4 + r] = acc[mb][r];
        if (q4 == 0) {
            sML[w][i16][0] = m_run;
            sML[w][i16][1] = l_run;
        }
    }
    __syncthreads();
    const int part = s / NWV;
    for (int x = threadIdx.x; x < G * D; x += NWV * 64) {
        const int g = x / D, d = x % D;
        float M = kNegInf;
#pragma unroll
        for (int w2 = 0; w2 < NWV; ++w2) M = fmaxf(M, sML[w2][g][0]);
        float o = 0.f, l = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w2 = 0; w2 < NWV; ++w2) {
                const float a = fast_exp2(sML[w2][g][0] - M);   // 0 for an empty split
                o += a * sRed[w2][g][d];
                l += a * sML[w2][g][1];
            }
        }
        const int64_t ix = ((int64_t)grp * p.npart + part) * G + g;
        p.part_o[ix * D + d] = o;
        if (d == 0) {
            p.part_ml[ix * 2 + 0] = M;
            p.part_ml[ix * 2 + 1] = l;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void mala_dec_dense_combine(const DecParams p) {
    __shared__ float sM[256];
    __shared__ float sO[8][32];
    __shared__ float sL[8];
    const int tid = threadIdx.x;
    const int grp = blockIdx.x, g = blockIdx.y, dq = blockIdx.z;
    const int G = p.G;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    const int nTb = (dec_len(p, b) + BKD - 1) / BKD;     // 0: skipped sequence
    const int64_t base = (int64_t)grp * p.npart;
    if (dq == 0 && g == 0) {
        if (tid == 0 && p.kept_tiles) p.kept_tiles[grp] = nTb;
        if (p.bits)
            for (int wd = tid; wd < p.nwords; wd += 256) {
                const int rem = nTb - 32 * wd;
                p.bits[(int64_t)grp * p.nwords + wd] =
                    rem >= 32 ? 0xFFFFFFFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
            }
    }
    if (nTb == 0) return;                         // o and lse are left as they were
    // global max over splits
    float mx = kNegInf;
    for (int s = tid; s < p.npart; s += 256) mx = fmaxf(mx, p.part_ml[((base + s) * G + g) * 2]);
    sM[tid] = mx;
    __syncthreads();
    for (int off = 128; off >= 1; off >>= 1) {
        if (tid < off) sM[tid] = fmaxf(sM[tid], sM[tid + off]);
        __syncthreads();
    }
    const float M = sM[0];
    const int d = 32 * dq + (tid & 31), cls = tid >> 5;
    float osum = 0.f, lsum = 0.f;
#pragma unroll 4
    for (int s = cls; s < p.npart; s += 8) {
        const int64_t ix = (base + s) * G + g;
        const float ms = p.part_ml[ix * 2];
        const float a = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
        osum += p.part_o[(((int64_t)grp * p.npart + s) * G + g) * D + d] * a;
        lsum += p.part_ml[ix * 2 + 1] * a;
    }
    sO[cls][tid & 31] = osum;
    if ((tid & 31) == 0) sL[cls] = lsum;
    __syncthreads();
    if (tid < 32) {
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) { o += sO[c][tid]; l += sL[c]; }
        p.o[((int64_t)b * p.Hq + kh * G + g) * D + 32 * dq + tid] = (uint16_t)float_to_bf16_bits(o / l);
        if (dq == 0 && tid == 0) p.lse[(int64_t)b * p.Hq + kh * G + g] = (M + fast_log2(l)) * kLn2;
    }
}

template <int D, int GP>
static hipError_t launch_decode_t(const DecParams& p, bool dense, hipStream_t s) {
    const int ngrp = p.B * p.Hkv;
    if (dense) {
        // one wave per (group, split); nsplit is a multiple of 8
        hipLaunchKernelGGL((mala_dec_dense<D, GP>), dim3(ngrp * p.nsplit / 8), dim3(512), 0, s, p);
        hipLaunchKernelGGL((mala_dec_dense_combine<D>), dim3(ngrp, p.G, D / 32), dim3(256), 0, s, p);
    } else {
        const int tasks = ngrp * p.nT;
        int nwg = (tasks + kScoreWaves - 1) / kScoreWaves;
        if (nwg > 256) nwg = 256;        // one workgroup (8 waves) per CU
        hipLaunchKernelGGL((mala_dec_score<D, GP>), dim3(nwg), dim3(64 * kScoreWaves), 0, s, p);
        hipLaunchKernelGGL((mala_dec_decide<GP>), dim3(ngrp), dim3(512), 0, s, p);
        hipLaunchKernelGGL((mala_dec_pv<D, GP>), dim3(p.npv), dim3(256), 0, s, p);
        hipLaunchKernelGGL((mala_dec_sum_combine<D>), dim3(ngrp, p.G, D / 32), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecParams& p, bool dense, hipStream_t s) {
    if (p.G <= 1) return launch_decode_t<D, 1>(p, dense, s);
    if (p.G <= 2) return launch_decode_t<D, 2>(p, dense, s);
    if (p.G <= 4) return launch_decode_t<D, 4>(p, dense, s);
    if (p.G == 5) return launch_decode_t<D, 5>(p, dense, s);    // 40q / 8kv head models
    if (p.G <= 8) return launch_decode_t<D, 8>(p, dense, s);
    return launch_decode_t<D, 16>(p, dense, s);
}

hipError_t launch_decode(const DecParams& p, int d, int Bkd, bool dense, hipStream_t s) {
    if (Bkd != BKD || p.G > 16) return hipErrorInvalidValue;
    if (d == 128) return launch_decode_d<128>(p, dense, s);
    if (d == 64) return launch_decode_d<64>(p, dense, s);
    return hipErrorInvalidValue;
}

}  // namespace mala
