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
//                    tiles with the next tile's K fragments loaded into
//                    registers while the current tile is scored: S^T = K q^T
//                    with 32x32x16 bf16 MFMAs (the G rows padded to 32
//                    columns).  Writes per-row tile max and shifted sum and the
//                    base-2 scores (spill).  Reads every K byte once: the
//                    HBM-bound score discovery.
//   mala_dec_decide  one wave per (sequence, KV head): the sequential rule,
//                    evaluated 64 tiles per round.  The candidate set is every
//                    tile that votes keep under the state at the start of the
//                    round; an exact log-sum-exp prefix scan gives each tile the
//                    retained mass it would see if all earlier candidates are
//                    kept.  Candidates that still vote keep up to the first one
//                    that flips to skip are final (their prefixes were exact);
//                    the flipped tile is skipped and the next round starts after
//                    it.  A tile that votes skip under a smaller retained mass
//                    can never turn to keep, so non-candidates are final too.
//   mala_dec_pv      kept tiles only, one wave per tile: P = 2^(s - lse) from
//                    the spill, V rows loaded at once, fp32 accumulation, one
//                    partial output per workgroup of four tiles.
//   mala_dec_sum_combine  sums the partials (already normalised) -> bf16 o.
// tau = 0 keeps every tile, so the scan is elided: mala_dec_dense is a fused
// split-K decode (scores, online softmax and P.V per split) and
// mala_dec_dense_combine merges the splits.
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {

namespace {
constexpr int BKD = 64;

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

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mala_dec_score(const DecParams p) {
    constexpr int KSTEPS = D / 16;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    // Each wave streams a contiguous run of tiles.  K fragments (A operands:
    // row = key, 8 consecutive d) are loaded straight into registers, the next
    // tile's loads in flight while the current tile is scored; no LDS.
    const int ntask = p.B * p.Hkv * p.nT;
    const int nwave = gridDim.x * 4;
    const int per = (ntask + nwave - 1) / nwave;
    // wave-uniform, so the per-tile index arithmetic below runs on the scalar unit
    const int gw = __builtin_amdgcn_readfirstlane(w * gridDim.x + blockIdx.x);   // neighbouring runs on different CUs
    int task = gw * per;
    const int tend = (task + per < ntask) ? task + per : ntask;
    if (task >= tend) return;

    auto load_tile = [&](int tk, bf16x8 (&kf)[2][KSTEPS]) {
        const int grp = tk / p.nT, t = tk % p.nT;
        const int b = grp / p.Hkv, kh = grp % p.Hkv;
        const int Nb = dec_len(p, b);
        if (t * BKD >= Nb) return;                     // past this sequence's cache
        const uint16_t* kb = p.k + b * p.k_sb + kh * p.k_sh;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            int j = t * BKD + 32 * sub + l32;
            j = j < Nb ? j : Nb - 1;                   // rows past Nb are masked below
            const uint16_t* row = kb + (int64_t)j * p.k_sl + 8 * hi;
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) kf[sub][st] = *(const bf16x8*)(row + 16 * st);
        }
    };
    int qgrp = -1;
    bf16x8 qf[D / 16];
    auto score_tile = [&](int tk, const bf16x8 (&kf)[2][KSTEPS]) {
        const int grp = tk / p.nT;
        const int t = tk % p.nT;
        if (grp != qgrp) {
            load_q_frags<D>(p, grp / p.Hkv, grp % p.Hkv, qf);
            qgrp = grp;
        }
        // per-call reset owned by this tile
        if (p.bits && lane == 0 && (t % 32) == 0) p.bits[(int64_t)grp * p.nwords + t / 32] = 0u;
        const int Nb = dec_len(p, grp / p.Hkv);
        if (t * BKD >= Nb) return;
        f32x16 sv[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            sv[sub] = f32x16{};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) sv[sub] = mfma32x32x16(kf[sub][st], qf[st], sv[sub]);
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = t * BKD + 32 * sub + 8 * (r >> 2) + 4 * hi + (r & 3);
                sv[sub][r] = (j < Nb) ? sv[sub][r] * p.scale_log2 : kNegInf;
            }
        float M = kNegInf;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) M = fmaxf(M, sv[sub][r]);
        M = wave_max_pair(M);
        float sum = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += fast_exp2(sv[sub][r] - M);
        sum = wave_sum_pair(sum);
        const int g = l32;
        if (g < p.G) {
            float* sp = p.spill + ((int64_t)grp * p.G + g) * p.N + (int64_t)t * BKD;
            const bool full = (t + 1) * BKD <= Nb;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int j0 = 32 * sub + 8 * q4 + 4 * hi;
                    if (full) {
                        *(f32x4*)(sp + j0) =
                            f32x4{sv[sub][4 * q4], sv[sub][4 * q4 + 1], sv[sub][4 * q4 + 2], sv[sub][4 * q4 + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (t * BKD + j0 + e < Nb) sp[j0 + e] = sv[sub][4 * q4 + e];
                    }
                }
            if (hi == 0) {
                p.tmax[((int64_t)grp * p.G + g) * p.nTp + t] = M;
                p.tsum[((int64_t)grp * p.G + g) * p.nTp + t] = sum;
            }
        }
    };

    bf16x8 ka[2][KSTEPS], kb[2][KSTEPS];
    load_tile(task, ka);
    for (; task < tend; task += 2) {
        if (task + 1 < tend) load_tile(task + 1, kb);
        score_tile(task, ka);
        if (task + 1 < tend) {
            if (task + 2 < tend) load_tile(task + 2, ka);
            score_tile(task + 1, kb);
        }
    }
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

// The sequential decode rule with one wave per q head of the group (lane =
// tile, 64 tiles per chunk, newest first).  Same rounds, votes and prefix
// sums as the single-wave form, taken per row: each wave scans only its own
// row's linear masses, and the rows meet through two 64-bit masks per round
// in LDS (the candidates: some row votes keep; the survivors: some row still
// votes keep after the earlier candidates' mass), so a round is a few dozen
// instructions per wave instead of a loop over every row.  Runs when every
// row's tile maxima lie within 96 of its largest and tau/N within 2^+-120
// (the linear range); otherwise the first wave runs the single-wave form.
// Groups of more than 8 rows run the single-wave form on one wave (16 waves
// would leave the single-wave form too few registers).
template <int GP>
constexpr int decide_threads() { return GP <= 8 ? 64 * GP : 64; }

// Workgroup barrier after this wave's LDS writes have completed.  Unlike
// __syncthreads() it does not wait for vector-memory operations, so the
// statistics copies in flight (several chunks ahead) and the tile-list stores
// stay in flight across the barrier.  The scheduling barriers keep every LDS
// access on its side.
__device__ __forceinline__ void lds_only_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    // gfx9 s_waitcnt: lgkmcnt(0), vmcnt and expcnt at their maxima (no wait)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int GP>
__global__ __launch_bounds__(decide_threads<GP>()) void mala_dec_decide(const DecParams p) {
    const int grp = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int G = p.G;
    const int Nb = dec_len(p, grp / p.Hkv);
    if (Nb == 0) {                              // skipped sequence: nothing retained
        if (threadIdx.x == 0) {
            p.kcount[grp] = 0;
            if (p.kept_tiles) p.kept_tiles[grp] = 0;
        }
        return;
    }
    if constexpr (GP > 8) {
        decide_one_wave<GP>(p, Nb);
        return;
    }
    const int nTb = (Nb + BKD - 1) / BKD;      // this sequence's tiles (p.nT is the stride)
    const float theta = p.log2_tau - (p.seqlens ? (float)log2((double)Nb) : p.log2_N);
    const bool lin_ok = theta >= -120.f && theta <= 120.f;
    const float cthr = fast_exp2(theta);
    const int nchunk = (nTb + 63) / 64;
    const bool row = w < G;                     // waves past G hold no row (they only meet the barriers)
    const float* tmax = p.tmax + ((int64_t)grp * G + (row ? w : 0)) * p.nTp;
    const float* tsum = p.tsum + ((int64_t)grp * G + (row ? w : 0)) * p.nTp;

    // This row's tile statistics stream through an LDS ring, DEPTH chunks
    // ahead: two 4-byte copies per chunk (max, sum), tile t_lo + i at entry i
    // (reads before tile 0 return 0; such lanes are invalid).
    constexpr int DEPTH = 8, RING = DEPTH + 1;
    __shared__ __attribute__((aligned(16))) float sRow[RING][2][GP][64];
    __shared__ int sLin[GP];
    __shared__ uint64_t sCand[2][GP], sKeep[2][GP];
    const __amdgpu_buffer_rsrc_t rmax = make_rsrc(tmax, (uint32_t)(p.nTp * 4));
    const __amdgpu_buffer_rsrc_t rsum = make_rsrc(tsum, (uint32_t)(p.nTp * 4));
    auto issue_row = [&](int c) {
        const int t = nTb - 64 * (c + 1) + lane;
        const uint32_t off = (t >= 0) ? (uint32_t)(t * 4) : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rmax, (__attribute__((address_space(3))) void*)(&sRow[c % RING][0][w][0]),
                                                4, (int)off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsum, (__attribute__((address_space(3))) void*)(&sRow[c % RING][1][w][0]),
                                                4, (int)off, 0, 0, 0);
    };
    if (row)
        for (int c = 0; c < DEPTH && c < nchunk; ++c) issue_row(c);

    // Row reference: the largest tile max; the row is in the linear range when
    // its smallest tile max lies within 96 of it.  16-byte loads, 8 per lane
    // issued together, branch-free (indexes past the row re-read entry 0).
    float gref = 0.f;
    {
        bool lin = true;
        if (row) {
            float mx = kNegInf, mn = __builtin_inff();
            const int nq = nTb >> 2;
            for (int j0 = 0; j0 < nq; j0 += 64 * 8) {
                f32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = j0 + 64 * u + lane;
                    v[u] = *(const f32x4*)(tmax + 4 * (j < nq ? j : 0));
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const bool ok = j0 + 64 * u + lane < nq;
                    const float a = fmaxf(fmaxf(v[u][0], v[u][1]), fmaxf(v[u][2], v[u][3]));
                    const float b = fminf(fminf(v[u][0], v[u][1]), fminf(v[u][2], v[u][3]));
                    mx = ok ? fmaxf(mx, a) : mx;
                    mn = ok ? fminf(mn, b) : mn;
                }
            }
            const bool ok = lane < nTb - 4 * nq;
            const float v = tmax[ok ? 4 * nq + lane : 0];
            mx = ok ? fmaxf(mx, v) : mx;
            mn = ok ? fminf(mn, v) : mn;
            gref = wave_max_all(mx);
            const float lo = -wave_max_all(-mn);
            lin = lo >= gref - 96.f;
        }
        if (lane == 0) sLin[w] = lin ? 1 : 0;
    }
    __syncthreads();
    bool linear = lin_ok;
#pragma unroll
    for (int g = 0; g < GP; ++g) linear = linear && (sLin[g] != 0);
    if (!linear) {
        if (w == 0) decide_one_wave<GP>(p, Nb);
        return;
    }

    int32_t* klist = p.klist + (int64_t)grp * p.nT;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    float Z = row ? 0.f : 1.f;                  // retained mass of this row, relative to gref
    bool empty = true;                          // nothing retained yet: the next candidate is kept
    int kept = 0;
    int par = 0;                                // mask slots alternate between rounds
    for (int c = 0; c < nchunk; ++c) {
        const int t = nTb - 1 - (c * 64 + lane);
        const bool valid = t >= 0;
        float a = 0.f, x = 0.f;
        if (row) {
            if (c + DEPTH < nchunk) {
                issue_row(c + DEPTH);
                wait_vmcnt<2 * DEPTH>();                  // chunk c has landed
            } else {
                wait_vmcnt<0>();
            }
            const float M = sRow[c % RING][0][w][63 - lane];
            const float S = sRow[c % RING][1][w][63 - lane];
            a = valid ? fast_exp2(M - gref) : 0.f;
            x = valid ? S * a : 0.f;
        }
        int pos = 0;
        while (true) {
            const bool active = valid && lane >= pos;
            const uint64_t mine = __ballot(active && (a >= cthr * Z));
            if (lane == 0) sCand[par][w] = mine;
            lds_only_barrier();
            uint64_t K0 = 0ull;
#pragma unroll
            for (int g = 0; g < GP; ++g) K0 |= sCand[par][g];
            if (empty) K0 = __ballot(active);
            if (K0 == 0ull) {                             // the rest of the chunk is skipped
                par ^= 1;
                break;
            }
            const int first = __builtin_ctzll(K0);
            const bool cand = (K0 >> lane) & 1ull;
            const float inc = wave_incl_sum(cand ? x : 0.f);
            // the previous lane's inclusive sum, never inc minus this tile's mass
            const float exc = wave_shr1(inc);
            const uint64_t still = __ballot(cand && (a >= cthr * (Z + exc)));
            if (lane == 0) sKeep[par][w] = still;
            lds_only_barrier();
            uint64_t V1 = empty ? (1ull << first) : 0ull;
#pragma unroll
            for (int g = 0; g < GP; ++g) V1 |= sKeep[par][g];
            par ^= 1;
            const uint64_t flips = K0 & ~V1;
            uint64_t acc;
            if (flips == 0ull) {
                acc = K0;
                Z += readlane_f(inc, 63);
            } else {
                const int f = __builtin_ctzll(flips);
                acc = K0 & ((f == 0) ? 0ull : (~0ull >> (64 - f)));
                Z += readlane_f(exc, f);
                pos = f + 1;
            }
            if (w == 0 && ((acc >> lane) & 1ull)) {
                klist[kept + __builtin_popcountll(acc & lt_mask)] = t;
                if (p.bits) atomicOr(p.bits + (int64_t)grp * p.nwords + t / 32, 1u << (t % 32));
            }
            kept += __builtin_popcountll(acc);
            if (acc) empty = false;
            if (flips == 0ull) break;
        }
    }
    if (threadIdx.x == 0) {
        p.kcount[grp] = kept;
        if (p.kept_tiles) p.kept_tiles[grp] = kept;
    }
    if (row && lane == 0) {
        const float lz2 = gref + fast_log2(Z);
        p.lse2[(int64_t)grp * G + w] = lz2;
        const int b = grp / p.Hkv, kh = grp % p.Hkv;
        p.lse[(int64_t)b * p.Hq + kh * G + w] = lz2 * kLn2;
    }
}

// P.V over the kept tiles: one wave per kept tile, four per workgroup, every
// load issued at once (the tile index, then its V rows and spilled scores).
// Lane (dc, kg) owns d = 8 dc .. 8 dc + 7 of KPL consecutive keys; the wave's
// partial output is reduced across kg with lane shuffles, the workgroup's
// across its waves in LDS, and written as one partial per workgroup.
template <int D, int GP>
__global__ __launch_bounds__(256) void mala_dec_pv(const DecParams p) {
    constexpr int DC = D / 8;            // 16-byte chunks per V row
    constexpr int KG = 64 / DC;          // key groups per wave
    constexpr int KPL = BKD / KG;        // keys per lane
    __shared__ float sP[4][GP][BKD];
    __shared__ float sRed[4][GP][D];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int grp = blockIdx.y;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    const int G = p.G;
    const int idx = blockIdx.x * 4 + w;
    // the list entry is read together with the count (one round trip instead
    // of two); entries past the count are stale and not used
    const int tl = p.klist[(int64_t)grp * p.nT + (idx < p.nT ? idx : p.nT - 1)];
    const int cnt = p.kcount[grp];
    asm volatile("" ::"v"(tl));                 // keep the list load ahead of the count test
    if (blockIdx.x * 4 >= cnt) return;          // the whole workgroup: no partial is read
    const int Nb = dec_len(p, b);
    const bool has = idx < cnt;
    const int t = has ? tl : 0;
    const int dc = lane % DC, kg = lane / DC;
    // V rows of this lane's keys (16-byte chunk dc)
    u32x4 vx[KPL];
    const uint16_t* vb = p.v + b * p.v_sb + kh * p.v_sh + 8 * dc;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
        int key = t * BKD + kg * KPL + r;
        key = key < Nb ? key : Nb - 1;
        vx[r] = *(const u32x4*)(vb + (int64_t)key * p.v_sl);
    }
    __builtin_amdgcn_sched_barrier(0);          // the V loads go out first, then the P loads
    // P of the tile: lane = key, one value per row.  The loads take clamped
    // (always valid) indices and are issued together; invalid entries are
    // replaced by 0 afterwards.
    {
        const int key = t * BKD + lane;
        const bool kok = has && key < Nb;
        const int kk = kok ? key : 0;
        float sv[GP], lv[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const int gg = g < G ? g : G - 1;
            sv[g] = p.spill[((int64_t)grp * G + gg) * p.N + kk];
            lv[g] = p.lse2[(int64_t)grp * G + gg];
        }
#pragma unroll
        for (int g = 0; g < GP; ++g) sP[w][g][lane] = (kok && g < G) ? fast_exp2(sv[g] - lv[g]) : 0.f;
    }
    __syncthreads();
    float acc[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
#pragma unroll
    for (int r = 0; r < KPL; ++r) {
        float vv[8];
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) {
            vv[2 * m2] = __uint_as_float(vx[r][m2] << 16);
            vv[2 * m2 + 1] = __uint_as_float(vx[r][m2] & 0xFFFF0000u);
        }
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float pr = sP[w][g][kg * KPL + r];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] += pr * vv[e];
        }
    }
    // reduce over the key groups of the wave (lanes dc + DC * kg)
#pragma unroll
    for (int off = DC; off < 64; off <<= 1)
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], off);
    if (kg == 0) {
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) sRed[w][g][8 * dc + e] = acc[g][e];
    }
    __syncthreads();
    float* po = p.part_o + (((int64_t)grp * p.npart + blockIdx.x) * G) * D;
    for (int e = tid; e < G * D; e += 256) {
        const int g = e / D, d = e % D;
        po[e] = sRed[0][g][d] + sRed[1][g][d] + sRed[2][g][d] + sRed[3][g][d];
    }
}

// Sum of the P.V partials (already normalised by the final LSE) -> bf16 o.
// One workgroup per (group, row, 32-wide d slice): 8 split classes x 32 d.
template <int D>
__global__ __launch_bounds__(256) void mala_dec_sum_combine(const DecParams p) {
    __shared__ float sO[8][32];
    const int tid = threadIdx.x;
    const int grp = blockIdx.x, g = blockIdx.y, dq = blockIdx.z;
    const int G = p.G;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    if (dec_len(p, b) == 0) return;              // skipped sequence: o is left as it was
    const int64_t base = (int64_t)grp * p.npart;
    const int d = 32 * dq + (tid & 31), cls = tid >> 5;
    const int nused = (p.kcount[grp] + 3) / 4;   // P.V workgroups that wrote a partial
    float osum = 0.f;
#pragma unroll 4
    for (int s = cls; s < nused; s += 8) osum += p.part_o[((base + s) * G + g) * D + d];
    sO[cls][tid & 31] = osum;
    __syncthreads();
    if (tid < 32) {
        float o = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o += sO[c][tid];
        p.o[((int64_t)b * p.Hq + kh * G + g) * D + 32 * dq + tid] = (uint16_t)float_to_bf16_bits(o);
    }
}

// tau = 0: fused split-K decode.  Each workgroup owns tiles_per_split tiles of
// one (sequence, KV head); per round its 4 waves stage and score 4 tiles while
// every thread's V rows for those tiles are already in flight; then the
// online-softmax update and P.V for the 256 keys.
template <int D, int GP>
__global__ __launch_bounds__(256) void mala_dec_dense(const DecParams p) {
    constexpr int DC = D / 8;
    constexpr int NKG = 256 / DC;
    constexpr int KPT = 4 * BKD / NKG;
    __shared__ __attribute__((aligned(16))) uint16_t sK[4][BKD * D];
    __shared__ float sS[GP][4 * BKD];
    __shared__ float sAlpha[GP];
    __shared__ float sState[GP][2];      // running max, sum (base 2)
    __shared__ float sRed[NKG][D];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int s = blockIdx.x, grp = blockIdx.y;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    const int G = p.G;
    const int Nb = dec_len(p, b);
    const int nTb = (Nb + BKD - 1) / BKD;
    const int t0 = s * p.tiles_per_split;
    const int t1 = (t0 + p.tiles_per_split < nTb) ? t0 + p.tiles_per_split : nTb;   // may be empty
    bf16x8 qf[D / 16];
    load_q_frags<D>(p, b, kh, qf);
    if (tid < GP) { sState[tid][0] = kNegInf; sState[tid][1] = 0.f; }
    const int dc = tid % DC, kg = tid / DC;
    float acc[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    const uint16_t* vb = p.v + b * p.v_sb + kh * p.v_sh + 8 * dc;
    __syncthreads();
    for (int tb = t0; tb < t1; tb += 4) {
        const int t = tb + w;
        if (t < t1) stage_k_tile<D>(p, b, kh, t, Nb, sK[w]);
        u32x4 vx[KPT];
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            int key = tb * BKD + kg * KPT + r;
            key = (key < t1 * BKD && key < Nb) ? key : 0;
            vx[r] = *(const u32x4*)(vb + (int64_t)key * p.v_sl);
        }
        {
            f32x16 sc[2];
            if (t < t1) {
                __builtin_amdgcn_s_waitcnt(0);
                tile_scores<D>(p, t, Nb, sK[w], qf, sc);
            } else {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[sub][r] = kNegInf;
            }
            if (l32 < G) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        sS[l32][w * BKD + 32 * sub + 8 * (r >> 2) + 4 * hi + (r & 3)] = sc[sub][r];
            }
        }
        __syncthreads();
        // online softmax over the 256 new scores: 16 threads per row
        {
            const int g = tid >> 4, part = tid & 15;
            float mx = kNegInf;
            if (g < G)
                for (int j = part; j < 4 * BKD; j += 16) mx = fmaxf(mx, sS[g][j]);
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            float mo = kNegInf, lo = 0.f;
            if (g < G) { mo = sState[g][0]; lo = sState[g][1]; }
            const float mn = fmaxf(mo, mx);
            const float muse = (mn == kNegInf) ? 0.f : mn;
            float sum = 0.f;
            if (g < G)
                for (int j = part; j < 4 * BKD; j += 16) {
                    const float e = fast_exp2(sS[g][j] - muse);
                    sS[g][j] = e;
                    sum += e;
                }
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
            __syncthreads();
            if (g < G && part == 0) {
                const float a = (mo == kNegInf) ? 0.f : fast_exp2(mo - muse);
                sAlpha[g] = a;
                sState[g][0] = mn;
                sState[g][1] = lo * a + sum;
            }
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            if (g < G) {
                const float a = sAlpha[g];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] *= a;
            }
        }
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int jj = kg * KPT + r;
            const int key = tb * BKD + jj;
            if (key >= t1 * BKD || key >= Nb) continue;
            float vv[8];
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2) {
                vv[2 * m2] = __uint_as_float(vx[r][m2] << 16);
                vv[2 * m2 + 1] = __uint_as_float(vx[r][m2] & 0xFFFF0000u);
            }
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                if (g < G) {
                    const float pr = sS[g][jj];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[g][e] += pr * vv[e];
                }
            }
        }
        __syncthreads();
    }
    float* po = p.part_o + (((int64_t)grp * p.npart + s) * G) * D;
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int gg = 0; gg < GP; ++gg)
            if (gg == g)
#pragma unroll
                for (int e = 0; e < 8; ++e) sRed[kg][8 * dc + e] = acc[gg][e];
        __syncthreads();
        if (tid < D) {
            float sum = 0.f;
#pragma unroll
            for (int k2 = 0; k2 < NKG; ++k2) sum += sRed[k2][tid];
            po[(int64_t)g * D + tid] = sum;
        }
        __syncthreads();
    }
    if (tid < G) {
        p.part_ml[(((int64_t)grp * p.nsplit + s) * G + tid) * 2 + 0] = sState[tid][0];
        p.part_ml[(((int64_t)grp * p.nsplit + s) * G + tid) * 2 + 1] = sState[tid][1];
    }
}

// One workgroup per (group, row, 32-wide d slice): 8 split classes x 32 d.
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
    const int64_t base = (int64_t)grp * p.nsplit;
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
    for (int s = tid; s < p.nsplit; s += 256) mx = fmaxf(mx, p.part_ml[((base + s) * G + g) * 2]);
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
    for (int s = cls; s < p.nsplit; s += 8) {
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
        hipLaunchKernelGGL((mala_dec_dense<D, GP>), dim3(p.nsplit, ngrp), dim3(256), 0, s, p);
        hipLaunchKernelGGL((mala_dec_dense_combine<D>), dim3(ngrp, p.G, D / 32), dim3(256), 0, s, p);
    } else {
        const int tasks = ngrp * p.nT;
        int nwg = (tasks + 3) / 4;
        if (nwg > 512) nwg = 512;        // two workgroups (8 waves) per CU
        hipLaunchKernelGGL((mala_dec_score<D>), dim3(nwg), dim3(256), 0, s, p);
        hipLaunchKernelGGL((mala_dec_decide<GP>), dim3(ngrp), dim3(decide_threads<GP>()), 0, s, p);
        hipLaunchKernelGGL((mala_dec_pv<D, GP>), dim3((p.nT + 3) / 4, ngrp), dim3(256), 0, s, p);
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
