// MALA backward (gfx950): offline sparse probabilities with nested support.
//
// Rule ("MassAlloc Attention: Let Attention Allocate Its Own Compute"; review
// page, "Backward: offline sparse probabilities"; summary page, backward
// paragraph): the backward does not replay the forward's partial
// normalisers.  With the final log-normaliser LSE saved by the forward, tile
// (query block, key tile) is kept iff some row i with a legal key has
//     max_j s_ij - LSE_i >= log(tau) - log(i+1),
// i.e. its largest exact probability reaches tau / L_i.  Since the final
// normaliser is at least every partial one, every tile the forward skipped is
// skipped again; no mask is stored.  For kept tiles the standard softmax
// gradient is accumulated:
//     P = exp(S - LSE), dV += P^T dO, dP = dO V^T, dS = P (dP - D),
//     dK += scale dS^T Q, dQ += scale dS K,   D_i = dO_i . O_i.
//
// Kernels:
//   mala_bwd_pre    D_i, LSE_i in base 2, transposed copies of Q and dO (query
//                   positions permuted inside each 16-group to match the MFMA
//                   register order), zeroed dQ accumulator and statistics.
//   mala_bwd_kernel one workgroup per (batch, KV head, key tile of 64 keys),
//                   4 waves.  K and V fragments stay in registers; the kernel
//                   streams the query blocks of every q head of the group,
//                   newest block first, through a double-buffered LDS tile and
//                   recomputes S = Q K^T for each (every legal tile is scored).
//                   Wave w owns keys 32(w&1).. and half (w>>1) of the block's
//                   queries.  S is laid out with one key per lane and the
//                   block's queries in registers, so P^T and dS^T feed the dV
//                   and dK contractions straight from registers; dS also goes
//                   to LDS (query-major) for dQ = dS K.  dK/dV accumulate in
//                   registers over heads and blocks; dQ goes to an fp32
//                   accumulator with atomics.
//   mala_dq_convert fp32 dQ accumulator -> bf16 dQ.
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {

namespace {
constexpr int BK = 64;
constexpr int PRE_ROWS = 64;

__device__ __forceinline__ int qpos(int i) { return (i & ~15) | vt_pos16(i & 15); }
}  // namespace

template <int D, int BQ>
__global__ __launch_bounds__(256) void mala_bwd_pre(const BwdParams p) {
    constexpr int TROW = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[PRE_ROWS * TROW];
    __shared__ __attribute__((aligned(16))) uint16_t sD[PRE_ROWS * TROW];
    const int tid = threadIdx.x;
    const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int r0 = rb * PRE_ROWS;
    const int L = p.L;
    const int64_t bh = (int64_t)b * p.Hq + h;
    // D_i = dO_i . O_i, LSE in base 2 and minus the keep threshold on raw scores
    // (4 threads per row).  Rows past L get D = 0, LSE = 0 and -inf, so their
    // scores never vote; with tau = 0 every legal tile is kept and the term is 0.
    {
        const int r = tid >> 2, part = tid & 3;
        const int i = r0 + r;
        float acc = 0.f;
        if (i < L) {
            const uint16_t* orow = p.o + b * p.o_sb + (int64_t)i * p.o_sl + h * p.o_sh;
            const uint16_t* grow = p.dout + b * p.do_sb + (int64_t)i * p.do_sl + h * p.do_sh;
            for (int c = part * 8; c < D; c += 32) {
                const u32x4 a = *(const u32x4*)(orow + c);
                const u32x4 g = *(const u32x4*)(grow + c);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    acc += __uint_as_float(a[m] << 16) * __uint_as_float(g[m] << 16);
                    acc += __uint_as_float(a[m] & 0xFFFF0000u) * __uint_as_float(g[m] & 0xFFFF0000u);
                }
            }
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        if (part == 0) {
            const int64_t ri = bh * p.Lpad + i;
            if (i < L) {
                const float l2 = p.lse[bh * L + i] * kLog2e;
                p.rowd[ri] = acc;
                p.rowc[ri] = l2;
                p.rowt[ri] = (p.log2_tau == kNegInf)
                                 ? 0.f
                                 : -(l2 + (p.log2_tau - fast_log2((float)(i + 1)))) / p.scale_log2;
                if (p.kept_slots) p.kept_slots[bh * L + i] = 0;
            } else {
                p.rowd[ri] = 0.f;
                p.rowc[ri] = 0.f;
                p.rowt[ri] = kNegInf;
            }
        }
    }
    // stage Q and dO rows (zeros past L)
    constexpr int CH = D / 8;
    for (int idx = tid; idx < PRE_ROWS * CH; idx += 256) {
        const int r = idx / CH, c = idx % CH;
        const int i = r0 + r;
        u32x4 xq = {0, 0, 0, 0}, xg = {0, 0, 0, 0};
        if (i < L) {
            xq = *(const u32x4*)(p.q + b * p.q_sb + (int64_t)i * p.q_sl + h * p.q_sh + 8 * c);
            xg = *(const u32x4*)(p.dout + b * p.do_sb + (int64_t)i * p.do_sl + h * p.do_sh + 8 * c);
        }
        *(u32x4*)(&sQ[r * TROW + 8 * c]) = xq;
        *(u32x4*)(&sD[r * TROW + 8 * c]) = xg;
    }
    // zero the fp32 dQ accumulator rows [B][Hq][L][D]
    for (int idx = tid; idx < PRE_ROWS * D / 4; idx += 256) {
        const int r = idx / (D / 4), c = idx % (D / 4);
        const int i = r0 + r;
        if (i < L) *(f32x4*)(p.dq_acc + (bh * L + i) * D + 4 * c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // statistics owned by the query block starting in these rows
    if ((r0 % BQ) == 0) {
        const int qb = r0 / BQ;
        if (qb < p.nQB) {
            if (p.kept_tiles && tid == 0) p.kept_tiles[bh * p.nQB + qb] = 0;
            if (p.bits)
                for (int wd = tid; wd < p.nwords; wd += 256) p.bits[(bh * p.nQB + qb) * p.nwords + wd] = 0u;
        }
    }
    __syncthreads();
    // transposed writes: thread -> (d row, 8 consecutive positions)
    for (int idx = tid; idx < D * (PRE_ROWS / 8); idx += 256) {
        const int d = idx / (PRE_ROWS / 8), pg = idx % (PRE_ROWS / 8);
        uint32_t wq[4], wg[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p0 = 8 * pg + 2 * e;
            const int ra = qpos(p0), rb2 = qpos(p0 + 1);   // involution on 0..63
            wq[e] = (uint32_t)sQ[ra * TROW + d] | ((uint32_t)sQ[rb2 * TROW + d] << 16);
            wg[e] = (uint32_t)sD[ra * TROW + d] | ((uint32_t)sD[rb2 * TROW + d] << 16);
        }
        const int64_t off = (bh * D + d) * p.Lpad + r0 + 8 * pg;
        *(u32x4*)(p.qt + off) = u32x4{wq[0], wq[1], wq[2], wq[3]};
        *(u32x4*)(p.dot + off) = u32x4{wg[0], wg[1], wg[2], wg[3]};
    }
}

template <int D, int BQ>
__global__ __launch_bounds__(256) void mala_bwd_kernel(const BwdParams p) {
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int NQS = BQ / 32;         // query subtiles of the block
    constexpr int WSUB = NQS / 2;        // query subtiles per wave
    constexpr int QCH = D / 8;           // 16-byte chunks per Q row
    constexpr int SROW = BK + 8;         // LDS row of dS [query][key] and K^T [d][key]
    constexpr int QSLOTS = BQ * QCH;     // 16-byte chunks per Q block
    constexpr int QINST = QSLOTS / 256;  // global->LDS copies per lane per block
    constexpr int NBUF = 3;              // Q blocks in flight: current + two prefetched
    constexpr int QBYTES = NBUF * BQ * D * 2;
    constexpr int RBYTES = 2 * 2 * DT * 16 * 64 * 4;     // epilogue reduction
    constexpr int UBYTES = QBYTES > RBYTES ? QBYTES : RBYTES;
    static_assert(QINST * 256 == QSLOTS && WSUB >= 1, "shape");

    // Q blocks: [NBUF][BQ][D] bf16, 16-byte chunk c of row r stored at chunk c ^ (r % QCH)
    __shared__ __attribute__((aligned(16))) unsigned char sU[UBYTES];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[D * SROW];
    __shared__ __attribute__((aligned(16))) uint16_t sdS[BQ * SROW];
    // [buf][keep threshold on raw scores | lse2 | D][query]
    __shared__ __attribute__((aligned(16))) float sRow[NBUF][3][BQ];
    __shared__ int sFlag[2][4];
    uint16_t* sQ = reinterpret_cast<uint16_t*>(sU);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int kw = w & 1;
    const int qh = w >> 1;

    const int u = xcd_unit(blockIdx.x, p.chunk);
    if (u >= p.nunits) return;
    const int kt = u % p.nKT;               // key tiles in increasing order: longest first
    const int bk = u / p.nKT;
    const int b = bk / p.Hkv;
    const int kh = bk % p.Hkv;
    const int L = p.L;
    const int j0 = kt * BK;
    const int G = p.G;
    const float c2 = p.scale_log2;
    const bool keep_all = p.log2_tau == kNegInf;   // tau = 0: dense backward

    // ---- resident K and V fragments (B operands: column = key, 8 consecutive d)
    const int jme = j0 + 32 * kw + l32;
    bf16x8 kf[KSTEPS], vf[KSTEPS];
    {
        const bool ok = jme < L;
        const uint16_t* kr = p.k + b * p.k_sb + (int64_t)(ok ? jme : 0) * p.k_sl + kh * p.k_sh;
        const uint16_t* vr = p.v + b * p.v_sb + (int64_t)(ok ? jme : 0) * p.v_sl + kh * p.v_sh;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            const u32x4 a = ok ? *(const u32x4*)(kr + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            const u32x4 c = ok ? *(const u32x4*)(vr + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            kf[st] = __builtin_bit_cast(bf16x8, a);
            vf[st] = __builtin_bit_cast(bf16x8, c);
        }
    }
    // ---- K^T into LDS for the dQ contraction (natural key order)
    for (int idx = tid; idx < BK * QCH; idx += 256) {
        const int r = idx / QCH, c = idx % QCH;
        const int j = j0 + r;
        const u32x4 x = (j < L) ? *(const u32x4*)(p.k + b * p.k_sb + (int64_t)j * p.k_sl + kh * p.k_sh + 8 * c)
                                : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            sKt[(8 * c + 2 * m) * SROW + r] = (uint16_t)(x[m] & 0xFFFFu);
            sKt[(8 * c + 2 * m + 1) * SROW + r] = (uint16_t)(x[m] >> 16);
        }
    }

    f32x16 dv[DT], dk[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { dv[dt] = f32x16{}; dk[dt] = f32x16{}; }

    const int qb_lo = j0 / BQ;
    const int nqb = p.nQB - qb_lo;
    const int nsteps = G * nqb;

    // Step s covers q head kh*G + s / nqb and query block nQB-1 - s % nqb
    // (newest block first, so workgroups that start together read the same Q).
    // Per-lane byte offsets of this lane's 16-byte chunks inside a Q block
    // (row r, logical chunk c stored at physical chunk c ^ (r % QCH)).
    uint32_t qoff[QINST];
#pragma unroll
    for (int n = 0; n < QINST; ++n) {
        const int sl = (n * 4 + w) * 64 + lane;
        const int r = sl / QCH, pc = sl % QCH;
        const int c = pc ^ (r % QCH);
        qoff[n] = (uint32_t)((r * p.q_sl + 8 * c) * 2);
    }
    int f_h = kh * G, f_qb = p.nQB - 1;     // the step being fetched
    // issue the copies of one step's Q block and row terms into buffer `buf`
    auto fetch_advance = [&](int buf) {
        const int64_t bh = (int64_t)b * p.Hq + f_h;
        const int row0 = f_qb * BQ;
        const int nrow = (L - row0 < BQ) ? L - row0 : BQ;
        // row terms: waves 0..2 copy threshold / lse2 / D (BQ floats each)
        if (w < 3 && lane * 4 < BQ) {
            const float* src = (w == 0 ? p.rowt : (w == 1 ? p.rowc : p.rowd)) + bh * p.Lpad + row0;
            load16_to_lds(src + 4 * lane, &sRow[buf][w][0]);
        }
        // the block's rows through a buffer resource ending at row L-1, so the
        // rows past L read as zero without per-lane clamps
        const uint16_t* qblk = p.q + b * p.q_sb + (int64_t)row0 * p.q_sl + f_h * p.q_sh;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qblk, (uint32_t)(((nrow - 1) * p.q_sl + D) * 2));
        unsigned char* dst = sU + buf * (BQ * D * 2);
#pragma unroll
        for (int n = 0; n < QINST; ++n) buffer16_to_lds(rq, qoff[n], dst + (n * 4 + w) * 64 * 16);
        if (--f_qb < qb_lo) { f_qb = p.nQB - 1; ++f_h; }
    };

    if (nsteps > 0) fetch_advance(0);
    if (nsteps > 1) fetch_advance(1);
    wait_all_then_barrier();

    int h = kh * G, qb = p.nQB - 1;         // the step being computed
    int s = 0;
    f32x16 sc[WSUB];
    while (s < nsteps) {
        // ---- inner loop over steps whose tile is skipped: score recompute and
        // predicate only, nothing else live (the accumulators stay untouched)
        bool keep = false;
        int buf = 0;
        bool diag = false;
        for (;;) {
            buf = s % NBUF;
            const bool prefetch = s + 2 < nsteps;
            if (prefetch) fetch_advance((s + 2) % NBUF);
            const uint16_t* sQb = sQ + buf * BQ * D;
            diag = (qb == qb_lo);
            // S' = Q K^T - threshold for the wave's query subtiles x 32 keys: the
            // accumulator starts at minus each row's threshold (row terms in LDS)
#pragma unroll
            for (int t = 0; t < WSUB; ++t) {
                const int qsub = WSUB * qh + t;
                const int row = 32 * qsub + l32;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 tv = *(const f32x4*)(&sRow[buf][0][32 * qsub + 8 * g4 + 4 * hi]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sc[t][4 * g4 + e] = tv[e];
                }
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    const int pc = (2 * st + hi) ^ (row % QCH);
                    const bf16x8 a = *(const bf16x8*)(&sQb[row * D + 8 * pc]);
                    sc[t] = mfma32x32x16(a, kf[st], sc[t]);
                }
            }
            // nested predicate: keep iff some legal (i, j) has S'_ij >= 0
            float mx = kNegInf;
            if (diag) {
#pragma unroll
                for (int t = 0; t < WSUB; ++t) {
                    const int qsub = WSUB * qh + t;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int ig = qb * BQ + 32 * qsub + 8 * (r >> 2) + 4 * hi + (r & 3);
                        mx = fmaxf(mx, (jme <= ig) ? sc[t][r] : kNegInf);
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < WSUB; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
            }
            const bool vote = keep_all || mx >= 0.f;
            const bool wave_any = __ballot(vote) != 0ull;
            if (lane == 0) sFlag[s & 1][w] = wave_any ? 1 : 0;
            // the block of step s+1 (copied during step s-1) must have landed; the
            // copies of step s+2 (QINST, plus one row-term copy on waves 0..2)
            // may stay in flight
            if (!prefetch) wait_vmcnt<0>();
            else if (w < 3) wait_vmcnt<QINST + 1>();
            else wait_vmcnt<QINST>();
            __syncthreads();
            keep = (sFlag[s & 1][0] | sFlag[s & 1][1] | sFlag[s & 1][2] | sFlag[s & 1][3]) != 0;
            if (keep) break;
            if (--qb < qb_lo) { qb = p.nQB - 1; ++h; }
            if (++s >= nsteps) break;
        }
        if (!keep) break;
        const int64_t bh = (int64_t)b * p.Hq + h;
        {
            // ---- dP = dO V^T (A operand rows straight from global dO)
            f32x16 dp[WSUB];
#pragma unroll
            for (int t = 0; t < WSUB; ++t) {
                const int qsub = WSUB * qh + t;
                const int i = qb * BQ + 32 * qsub + l32;
                const bool ok = i < L;
                const uint16_t* grow = p.dout + b * p.do_sb + (int64_t)(ok ? i : 0) * p.do_sl + h * p.do_sh;
                dp[t] = f32x16{};
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    const u32x4 x = ok ? *(const u32x4*)(grow + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
                    dp[t] = mfma32x32x16(__builtin_bit_cast(bf16x8, x), vf[st], dp[t]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // ---- P, dS; A operands (key rows x 8 permuted query positions) for dV, dK
            bf16x8 pa[2 * WSUB], da[2 * WSUB];
#pragma unroll
            for (int t = 0; t < WSUB; ++t) {
                const int qsub = WSUB * qh + t;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ql = 32 * qsub + 8 * g4 + 4 * hi;
                    const f32x4 tv = *(const f32x4*)(&sRow[buf][0][ql]);
                    const f32x4 lv = *(const f32x4*)(&sRow[buf][1][ql]);
                    const f32x4 dd = *(const f32x4*)(&sRow[buf][2][ql]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g4 + e;
                        const int ig = qb * BQ + ql + e;
                        const bool legal = (jme <= ig) && (ig < L);
                        const float pr = legal ? fast_exp2(__builtin_fmaf(sc[t][r] - tv[e], c2, -lv[e])) : 0.f;
                        const float ds = pr * (dp[t][r] - dd[e]);
                        pa[2 * t + (r >> 3)][r & 7] = to_bf16(pr);
                        const __bf16 dsb = to_bf16(ds);
                        da[2 * t + (r >> 3)][r & 7] = dsb;
                        sdS[(ql + e) * SROW + 32 * kw + l32] = __builtin_bit_cast(uint16_t, dsb);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // ---- dV += P^T dO, dK += dS^T Q  (B operands from the transposed copies)
            const int64_t tbase = (int64_t)bh * D * p.Lpad + qb * BQ + (BQ / 2) * qh + 8 * hi;
#pragma unroll
            for (int ks = 0; ks < 2 * WSUB; ++ks) {
                bf16x8 bg[DT], bq[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int64_t off = tbase + (int64_t)(32 * dt + l32) * p.Lpad + 16 * ks;
                    bg[dt] = __builtin_bit_cast(bf16x8, *(const u32x4*)(p.dot + off));
                    bq[dt] = __builtin_bit_cast(bf16x8, *(const u32x4*)(p.qt + off));
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    dv[dt] = mfma32x32x16(pa[ks], bg[dt], dv[dt]);
                    dk[dt] = mfma32x32x16(da[ks], bq[dt], dk[dt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();   // dS complete in LDS
            // ---- dQ += scale dS K, work items (query subtile, d tile) spread over the waves
            {
                float* dqblk = p.dq_acc + (bh * L + qb * BQ) * D;
                for (int item = w; item < NQS * DT; item += 4) {
                    const int qsub = item / DT, dt = item % DT;
                    f32x16 acc = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < BK / 16; ++ks) {
                        const bf16x8 a = *(const bf16x8*)(&sdS[(32 * qsub + l32) * SROW + 16 * ks + 8 * hi]);
                        const bf16x8 bb = *(const bf16x8*)(&sKt[(32 * dt + l32) * SROW + 16 * ks + 8 * hi]);
                        acc = mfma32x32x16(a, bb, acc);
                    }
                    // C[i = query][j = d]: lane = d, registers = queries
                    float* col = dqblk + 32 * dt + l32;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qq = 32 * qsub + 8 * (r >> 2) + 4 * hi + (r & 3);
                        if (qb * BQ + qq < L) unsafeAtomicAdd(col + (int64_t)qq * D, acc[r] * p.scale);
                    }
                }
            }
            // ---- statistics of the backward's own decisions
            if (tid == 0) {
                if (p.kept_tiles) atomicAdd(p.kept_tiles + bh * p.nQB + qb, 1);
                if (p.bits) atomicOr(p.bits + (bh * p.nQB + qb) * p.nwords + (kt >> 5), 1u << (kt & 31));
            }
            if (p.kept_slots && tid < BQ) {
                const int i = qb * BQ + tid;
                const int last = i - j0;
                if (i < L && last >= 0) atomicAdd(p.kept_slots + bh * L + i, (last < BK - 1 ? last : BK - 1) + 1);
            }
        }
        if (--qb < qb_lo) { qb = p.nQB - 1; ++h; }
        ++s;
    }

    // ---- epilogue: combine the two query halves, write dK (scaled) and dV
    __syncthreads();
    float* red = reinterpret_cast<float*>(sU);
    if (qh == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                red[(((kw * 2 + 0) * DT + dt) * 16 + r) * 64 + lane] = dv[dt][r];
                red[(((kw * 2 + 1) * DT + dt) * 16 + r) * 64 + lane] = dk[dt][r];
            }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dv[dt][r] += red[(((kw * 2 + 0) * DT + dt) * 16 + r) * 64 + lane];
                dk[dt][r] += red[(((kw * 2 + 1) * DT + dt) * 16 + r) * 64 + lane];
            }
        // C[i = key][j = d]: lane = d, registers = keys 8(r/4) + 4hi + r%4
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = j0 + 32 * kw + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (j < L) {
                    const int d = 32 * dt + l32;
                    p.dv[b * p.dv_sb + (int64_t)j * p.dv_sl + kh * p.dv_sh + d] =
                        (uint16_t)float_to_bf16_bits(dv[dt][r]);
                    p.dk[b * p.dk_sb + (int64_t)j * p.dk_sl + kh * p.dk_sh + d] =
                        (uint16_t)float_to_bf16_bits(dk[dt][r] * p.scale);
                }
            }
    }
}

template <int D>
__global__ __launch_bounds__(256) void mala_dq_convert(const BwdParams p) {
    const int64_t n = (int64_t)p.B * p.Hq * p.L * (D / 8);
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
        const int c = (int)(idx % (D / 8));
        const int64_t row = idx / (D / 8);
        const int i = (int)(row % p.L);
        const int64_t bh = row / p.L;
        const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
        const float* src = p.dq_acc + row * D + 8 * c;
        const f32x4 a = *(const f32x4*)src, bb = *(const f32x4*)(src + 4);
        u32x4 o;
        o[0] = float_to_bf16_bits(a[0]) | (float_to_bf16_bits(a[1]) << 16);
        o[1] = float_to_bf16_bits(a[2]) | (float_to_bf16_bits(a[3]) << 16);
        o[2] = float_to_bf16_bits(bb[0]) | (float_to_bf16_bits(bb[1]) << 16);
        o[3] = float_to_bf16_bits(bb[2]) | (float_to_bf16_bits(bb[3]) << 16);
        *(u32x4*)(p.dq + b * p.dq_sb + (int64_t)i * p.dq_sl + h * p.dq_sh + 8 * c) = o;
    }
}

template <int D, int BQ>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL((mala_bwd_pre<D, BQ>), dim3(p.Lpad / PRE_ROWS, p.Hq, p.B), dim3(256), 0, s, p);
    const int per = 8 * p.chunk;
    const int grid = (p.nunits + per - 1) / per * per;
    hipLaunchKernelGGL((mala_bwd_kernel<D, BQ>), dim3(grid), dim3(256), 0, s, p);
    const int64_t n = (int64_t)p.B * p.Hq * p.L * (D / 8);
    int cg = (int)((n + 255) / 256);
    if (cg > 8192) cg = 8192;
    hipLaunchKernelGGL((mala_dq_convert<D>), dim3(cg), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, int Bq, int Bk, hipStream_t s) {
    if (d == 128 && Bq == 128 && Bk == 64) return launch_bwd_t<128, 128>(p, s);
    if (d == 64 && Bq == 64 && Bk == 64) return launch_bwd_t<64, 64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace mala
