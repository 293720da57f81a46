// MALA forward: fused causal attention with post-score tile skipping (gfx950).
//
// Rule ("MassAlloc Attention: Let Attention Allocate Its Own Compute"; review
// page, "Forward: online sparse softmax"; summary page, forward paragraph):
// every legal key tile is scored; the block of Bq query rows keeps the tile
// when some row with a legal key either has no retained mass yet or has
//     tile_row_max - running_max - log(retained_sum) >= log(tau) - log(i+1),
// i.e. exp(tile row max) / retained mass >= tau / L_i.  A kept tile gets the
// online-softmax update, the V load and the P.V product; a skipped tile gets
// none of them and leaves the row state untouched.  Tiles go from the diagonal
// toward key 0.  The final log-normaliser is written as LSE.
//
// Work decomposition: one workgroup per (batch, q head, query block) with
// Bq/32 waves; wave w owns query rows 32w..32w+31 of the block and computes
// the transposed score tile S^T = K Q^T with 32x32x16 bf16 MFMAs, so every
// lane holds all scores of one query (16 keys per 32-key subtile, the other 16
// in lane l^32).  Row reductions are therefore in-lane plus one swap, the
// block decision is a wave ballot plus an LDS OR, and P^T feeds the next
// contraction O^T += V^T P^T straight from the score registers.
//   - Q fragments live in registers for the whole loop.
//   - K and V tiles move global -> LDS with direct copies (no registers),
//     16-byte chunks XOR-swizzled per row so the MFMA reads are conflict-free.
//   - V is read from an fp16 copy made once per call (exact for |v| <= 65504);
//     its MFMA operand (8 consecutive keys per lane for one d) comes from the
//     LDS transposing read ds_read_b64_tr_b16.  P.V is an fp16 contraction: P
//     in [0, 1] rounded to nearest fp16 keeps the relative weight error near
//     3e-4 (bf16 P would cost ~1e-3 on diffuse rows, as much as the bf16
//     rounding of O itself).
//   - Software pipeline: the keep decision of tile t needs only the row
//     statistics (m, l), not the accumulator, so the P.V of tile t runs one
//     iteration later; the V copy of tile t is issued after the score MFMAs of
//     tile t-1 and lands during the rest of the tile, and K(t-2) is fetched
//     while tile t-1 is scored.
//   - Causal masking only on diagonal (or ragged) tiles; the 1/sqrt(d) scale
//     is folded into the exponent's FMA; the accumulator is rescaled only when
//     some row's running max moved.
#include <type_traits>

#include "mala_device.h"
#include "mala_internal.h"

namespace mala {

namespace {
// One 64-key tile of V, bf16 rows (key j at src + j * src_stride, j < nvalid)
// -> fp16, transposed: dst[d * BK + pos] holds key (pos & ~15) | vt_pos16(pos & 15)
// of column d, zero for keys past nvalid.  Within each group of 16 keys the
// order is the one the P.V contraction consumes, so that one 16-byte read
// (8 positions) gives a lane exactly the 8 keys its P fragment holds.  The
// tile passes through LDS: coalesced 16-byte reads of whole rows, and
// coalesced 16-byte writes of whole transposed rows.
template <int D, int BK>
__device__ __forceinline__ void v_tile_to_f16t(const uint16_t* src, int64_t src_stride, int nvalid,
                                               uint16_t* dst, uint16_t (*sT)[D + 8]) {
    constexpr int CH = D / 8;
    for (int q = threadIdx.x; q < BK * CH; q += 256) {
        const int j = q / CH, c = q % CH;
        u32x4 o = {0, 0, 0, 0};
        if (j < nvalid) {
            const u32x4 x = *(const u32x4*)(src + (int64_t)j * src_stride + 8 * c);
#pragma unroll
            for (int m = 0; m < 4; ++m) o[m] = pack2_f16_from_f32bits(x[m] << 16, x[m] & 0xFFFF0000u);
        }
        *(u32x4*)(&sT[j][8 * c]) = o;
    }
    __syncthreads();
    for (int q = threadIdx.x; q < D * (BK / 8); q += 256) {
        const int d = q / (BK / 8), c = q % (BK / 8);
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int pos = 8 * c + e;
            h[e] = sT[(pos & ~15) | vt_pos16(pos & 15)][d];
        }
        const u32x4 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        *(u32x4*)(dst + d * BK + 8 * c) = o;
    }
    __syncthreads();                             // sT is reused by the next tile
}

// V copy: bf16 [B, L, Hkv, D] -> fp16 [B, Hkv, Lpad / BK tiles, D, BK], each
// tile transposed as above; keys past L are zero.  One workgroup per tile.
template <int D, int BK>
__global__ __launch_bounds__(256) void mala_v_to_f16(const FwdParams p) {
    if (blockIdx.x == 0 && threadIdx.x < 8) p.queue[threadIdx.x] = 0;   // the forward's work queues
    __shared__ __attribute__((aligned(16))) uint16_t sT[BK][D + 8];
    const int ntile = p.Lpad / BK;
    const int64_t n = (int64_t)p.B * p.Hkv * ntile;
    for (int64_t u = blockIdx.x; u < n; u += gridDim.x) {
        const int t = (int)(u % ntile);
        const int64_t bk = u / ntile;
        const int kh = (int)(bk % p.Hkv), b = (int)(bk / p.Hkv);
        const int j0 = t * BK;
        v_tile_to_f16t<D, BK>(p.v + b * p.v_sb + (int64_t)j0 * p.v_sl + kh * p.v_sh, p.v_sl, p.L - j0,
                              p.vh + (bk * p.Lpad + j0) * D, sT);
    }
}

// Sequence b of a packed batch: row offsets and counts, or false when its
// cumulative lengths are inconsistent with the call's totals and maxima
// (such a sequence is left untouched).
struct SeqSpan {
    int q0, k0, Lq, Lk;
};
__device__ __forceinline__ bool seq_span(const FwdParams& p, int b, SeqSpan& s) {
    s.q0 = p.cu_q[b];
    s.k0 = p.cu_k[b];
    const int q1 = p.cu_q[b + 1], k1 = p.cu_k[b + 1];
    s.Lq = q1 - s.q0;
    s.Lk = k1 - s.k0;
    return s.q0 >= 0 && s.k0 >= 0 && q1 <= p.total_q && k1 <= p.total_k && s.Lq >= 0 && s.Lk >= s.Lq &&
           s.Lq <= p.max_q && s.Lk <= p.max_k;
}

// V copy of a packed batch: bf16 [total_k, Hkv, D] -> fp16 [Hkv, Rk, D] rows,
// sequence b's keys starting at row cu_k[b] + b * BK (at least BK spare rows
// follow each sequence).  From there its keys form transposed tiles as above;
// the last tile is zero past the sequence's keys.  grid.y = sequence.
template <int D, int BK>
__global__ __launch_bounds__(256) void mala_v_to_f16_varlen(const FwdParams p) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 8) p.queue[threadIdx.x] = 0;   // the forward's work queues
    __shared__ __attribute__((aligned(16))) uint16_t sT[BK][D + 8];
    const int b = blockIdx.y;
    SeqSpan sp;
    if (!seq_span(p, b, sp)) return;
    const int ntile = (sp.Lk + BK - 1) / BK;
    const int64_t n = (int64_t)p.Hkv * ntile;
    for (int64_t u = blockIdx.x; u < n; u += gridDim.x) {
        const int t = (int)(u % ntile);
        const int kh = (int)(u / ntile);
        const int j0 = t * BK;
        v_tile_to_f16t<D, BK>(p.v + (int64_t)(sp.k0 + j0) * p.v_sl + kh * p.v_sh, p.v_sl, sp.Lk - j0,
                              p.vh + ((int64_t)kh * p.Rk + sp.k0 + (int64_t)b * BK + j0) * D, sT);
    }
}
}  // namespace

template <int D, int BQ, int BK, bool STATS, bool VARLEN>
__global__ __launch_bounds__(BQ / 32 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mala_fwd_kernel(const FwdParams p) {
    constexpr int NW = BQ / 32;
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int QCH = D / 8;                   // 16-byte chunks per row
    constexpr int TILE_SLOTS = BK * QCH;         // 16-byte chunks per tile
    constexpr int INST = TILE_SLOTS / (NW * 64); // copies per lane per tile
    static_assert(BK == 64, "tile width");
    static_assert(INST * NW * 64 == TILE_SLOTS, "copy split");

    // K: [2][BK][D] bf16, chunk c of row r at c ^ (r % QCH)
    // V: [2][D][BK] fp16, a transposed tile of the V copy (row d, 8 key
    //    positions per 16-byte chunk), chunk c of row d at c ^ ((d / 2) % 8).
    //    A 16-byte read serves 16 lanes at a time over 64 banks, i.e. 16 rows
    //    d0..d0+15 of one chunk; rows of one parity share a 256-byte bank
    //    cycle, and the swizzle gives those 8 rows 8 different chunks.
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][BK * D];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][BK * D];
    __shared__ int sFlag[2][NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: w-derived addresses stay scalar
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // Persistent workgroups (eight waves per CU) take query blocks from eight queues,
    // one per XCD, each holding that XCD's share of the blocks in the launch
    // order below (longest first, chunks of blocks sharing K/V tiles together).
    // A workgroup drains its own XCD's queue, then the others'.  Blocks differ
    // in cost (kept tiles), and taking work from queues keeps every CU busy
    // where a launch of one workgroup per block would stall the in-order
    // dispatch behind the busiest XCD.
    __shared__ int sUnit;
    const int xcd = blockIdx.x & 7;
    int qsel = xcd;                              // next queue to draw from (thread 0)
    auto run_unit = [&](const int u) {
        const int nbh = p.B * p.Hq;
        const int qb = p.nQB - 1 - u / nbh;          // longest blocks first
        const int bh = u % nbh;
        const int b = bh / p.Hq;
        const int h = bh % p.Hq;
        const int kh = h / p.G;

        // The block's sequence: Lq queries that are the last Lq of its Lk keys
        // (Lq = Lk = L for the fixed-length layout), so query row i sees keys
        // j <= off + i and has L_i = off + i + 1 visible keys.
        int Lq, Lk;
        const uint16_t *qbase, *kbase, *vhbase;
        uint16_t* obase;
        int64_t rowbase;                             // lse / kept_slots / omitted index of row 0
        int64_t vh_rows;                             // rows of this KV head's fp16 V range
        if constexpr (VARLEN) {
            SeqSpan sp;
            const bool ok = seq_span(p, b, sp);
            Lq = ok ? sp.Lq : 0;
            Lk = sp.Lk;
            qbase = p.q + (int64_t)sp.q0 * p.q_sl + h * p.q_sh;
            obase = p.o + (int64_t)sp.q0 * p.o_sl + h * p.o_sh;
            kbase = p.k + (int64_t)sp.k0 * p.k_sl + kh * p.k_sh;
            vhbase = p.vh + ((int64_t)kh * p.Rk + sp.k0 + (int64_t)b * BK) * D;
            vh_rows = (int64_t)Lk + BK;
            rowbase = (int64_t)h * p.total_q + sp.q0;
        } else {
            Lq = Lk = p.L;
            qbase = p.q + b * p.q_sb + h * p.q_sh;
            obase = p.o + b * p.o_sb + h * p.o_sh;
            kbase = p.k + b * p.k_sb + kh * p.k_sh;
            vhbase = p.vh + ((int64_t)b * p.Hkv + kh) * p.Lpad * D;
            vh_rows = p.Lpad;
            rowbase = (int64_t)bh * p.L;
        }
        const int off = Lk - Lq;
        const int i0 = qb * BQ;
        if (i0 >= Lq) {
            // past the sequence's queries: nothing to visit (statistics read as such)
            if (tid == 0 && p.kept_tiles) p.kept_tiles[(int64_t)bh * p.nQB + qb] = 0;
            if (tid == 0 && p.bits)
                for (int wd = 0; wd < p.nwords; ++wd) p.bits[((int64_t)bh * p.nQB + qb) * p.nwords + wd] = 0u;
            return;
        }
        const int i = i0 + 32 * w + l32;             // this lane's query row
        const bool valid = i < Lq;
        const int ik = off + i;                      // its last visible key
        const int rend = (i0 + BQ < Lq) ? i0 + BQ : Lq;
        const int kt_first = (off + rend - 1) / BK;
        const bool ragged = (i0 + BQ > Lq);

        // ---- Q fragments (B operand: column = query, 8 consecutive d per lane)
        bf16x8 qf[KSTEPS];
        {
            const uint16_t* qrow = qbase + (int64_t)(valid ? i : 0) * p.q_sl;
    #pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                u32x4 x = valid ? *(const u32x4*)(qrow + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
                qf[st] = __builtin_bit_cast(bf16x8, x);
            }
        }

        // K and V tiles move global -> LDS through buffer resources with fixed
        // per-lane byte offsets.  K: one resource per tile, starting at the tile and
        // ending at key L-1, so rows past L read as zero (they are masked by
        // causality).  V: one resource over the padded fp16 copy, the tile offset
        // in a scalar (every access stays inside the copy).
        // V: copy n covers V^T rows NW * 64 / (BK / 8) further down than copy 0
        // with the same swizzle, so one lane offset serves every copy and the
        // rest goes into the scalar offset.
        uint32_t koff[INST];
    #pragma unroll
        for (int n = 0; n < INST; ++n) {
            const int sl = (n * NW + w) * 64 + lane;
            const int r = sl / QCH, pc = sl % QCH;
            koff[n] = (uint32_t)((r * p.k_sl + 8 * (pc ^ (r % QCH))) * 2);
        }
        constexpr uint32_t VSTEP = (uint32_t)(NW * 64 / (BK / 8)) * BK * 2;   // bytes between copies
        uint32_t voff;
        {
            const int sl = w * 64 + lane;
            const int dr = sl / (BK / 8), vc = sl % (BK / 8);
            voff = (uint32_t)((dr * BK + 8 * (vc ^ ((dr >> 1) & 7))) * 2);
        }
        static_assert((NW * 64) % ((BK / 8) * 16) == 0, "copy n keeps the V^T swizzle of copy 0");
        // The copies are issued from inline assembly (no compiler-inserted waits
        // before the reads of the other buffers); the wait before each barrier
        // covers them.
        const u32x4 vrs = raw_rsrc(vhbase, (uint32_t)(vh_rows * D * 2));
        auto copy_k = [&](int kt, int buf) {
            const int j0 = kt * BK;
            const u32x4 krs =
                raw_rsrc(kbase + (int64_t)j0 * p.k_sl, (uint32_t)(((int64_t)(Lk - 1 - j0) * p.k_sl + D) * 2));
    #pragma unroll
            for (int n = 0; n < INST; ++n)
                buffer16_to_lds_asm(krs, koff[n], 0u,
                                    reinterpret_cast<unsigned char*>(sK[buf]) + (n * NW + w) * 64 * 16);
        };
        auto copy_v = [&](int kt, int buf) {
            const uint32_t so = (uint32_t)(kt * BK * D * 2);
    #pragma unroll
            for (int n = 0; n < INST; ++n)
                buffer16_to_lds_asm(vrs, voff, so + n * VSTEP,
                                    reinterpret_cast<unsigned char*>(sV[buf]) + (n * NW + w) * 64 * 16);
        };
        // S^T = K Q^T for the tile in sK[buf]; raw (unscaled) scores
        auto scores = [&](int buf, f32x16* s) {
    #pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const int row = 32 * sub + l32;
                s[sub] = f32x16{};
    #pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    const int pc = (2 * st + hi) ^ (row % QCH);
                    const bf16x8 a = *(const bf16x8*)(&sK[buf][row * D + 8 * pc]);
                    s[sub] = mfma32x32x16(a, qf[st], s[sub]);
                }
            }
        };
        // causal mask (diagonal / ragged tiles) and raw row max
        auto mask_max = [&](int kt, f32x16* s) -> float {
            float M = kNegInf;
            const bool need = ragged || (kt * BK + BK - 1 > off + i0);
            if (need) {
                const int lim = valid ? (ik - kt * BK) : -1;
    #pragma unroll
                for (int sub = 0; sub < 2; ++sub)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int jj = 32 * sub + 8 * (r >> 2) + 4 * hi + (r & 3);
                        s[sub][r] = (jj <= lim) ? s[sub][r] : kNegInf;
                    }
            }
    #pragma unroll
            for (int sub = 0; sub < 2; ++sub)
    #pragma unroll
                for (int r = 0; r < 16; ++r) M = fmaxf(M, s[sub][r]);
            return wave_max_pair(M);
        };
        // V^T fragment of P.V step (dt, ks): row d = 32 dt + l32 of the
        // transposed tile, key positions 16 ks + 8 hi .. +7 (one 16-byte read)
        auto vt_frag = [&](const uint16_t* vbuf, int dt, int ks) -> f16x8 {
            const int dr = 32 * dt + l32;
            return *(const f16x8*)(vbuf + dr * BK + 8 * ((2 * ks + hi) ^ ((dr >> 1) & 7)));
        };
        // O^T += V^T P^T
        auto pv = [&](int buf, const f16x8* pb, f32x16* acc) {
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
    #pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc[dt] = mfma32x32x16_f16(vt_frag(sV[buf], dt, ks), pb[ks], acc[dt]);
            }
        };

        // ---- per-row state (this lane's query; lanes l and l^32 hold identical copies)
        const float c2 = p.scale_log2;
        float m2 = kNegInf;          // running max of retained base-2 scores
        float lsum = 0.f;            // retained sum, shifted by m2
        float thr = kNegInf;         // cached keep threshold m2 + log2(lsum) + theta
        const float theta = p.log2_tau - fast_log2((float)(ik + 1));
        float om = kNegInf, ol = 0.f;            // omitted mass (statistics mode)
        int slots = 0;
        f32x16 acc[DT];
    #pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

        int kept_count = 0;
        uint32_t bitword = 0;
        const bool want_bits = p.bits != nullptr;
        uint32_t* bitrow = want_bits ? p.bits + ((int64_t)bh * p.nQB + qb) * p.nwords : nullptr;
        if (want_bits && tid == 0) {
            for (int wd = kt_first / 32 + 1; wd < p.nwords; ++wd) bitrow[wd] = 0u;
        }

        // ---- prologue
        copy_k(kt_first, kt_first & 1);
        if (kt_first >= 1) copy_k(kt_first - 1, (kt_first - 1) & 1);
        wait_all_then_barrier();
        f32x16 sA[2], sB[2];         // scores: of the tile being decided / of the next tile
        f16x8 pp[4];                 // P of the pending tile, then of the tile being kept
        scores(kt_first & 1, sA);
        float Mraw = mask_max(kt_first, sA);

        bool pending = false;        // P.V of the last kept tile not yet accumulated
        int pend_buf = 0;
        float pend_alpha = 1.f;

        // One tile: decide tile kt from (m, l); then, in one straight-line block per
        // (keep, pending) case, issue the P.V MFMAs of the pending tile, then the
        // score MFMAs of tile kt-1 interleaved with the softmax of tile kt (whose P
        // reuses the registers the P.V just consumed).  The loop below runs two
        // tiles per iteration with the two score buffers in swapped roles, so
        // snext of one tile is scur of the next with no register copy.
        auto tile = [&](int kt, f32x16* scur, f32x16* snext) {
            const int buf = kt & 1;
            const float M = Mraw * c2;
            const bool has = Mraw > kNegInf;
            const bool vote = has && (lsum == 0.f || M >= thr);
            const bool wave_any = __ballot(vote) != 0ull;
            if (lane == 0) sFlag[buf][w] = wave_any ? 1 : 0;
            wait_all_then_barrier();                 // K(kt-1) and V of the pending tile have landed
            // The block's votes are read now but first used after the P.V of the
            // pending tile, which does not depend on them: the LDS round trip of
            // the read runs under that P.V.
            int kflag = 0;
    #pragma unroll
            for (int ww = 0; ww < NW; ++ww) kflag |= sFlag[buf][ww];

            if (kt >= 2) copy_k(kt - 2, buf);
            if (pending && __ballot(pend_alpha != 1.f) != 0ull) {
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= pend_alpha;
            }
            const uint16_t* kb = sK[buf ^ 1];        // K(kt-1); stale but harmless when kt == 0
            const uint16_t* vb = sV[pend_buf];
            // P.V of the pending tile (MFMA and LDS only).  Operand reads run two
            // MFMAs ahead through small register rings, and a scheduling barrier
            // closes every step, so the compiler keeps this order instead of
            // hoisting every LDS read.
            if (pending) {
                constexpr int NPV = 4 * DT;
                auto vread = [&](int s2) -> f16x8 { return vt_frag(vb, s2 % DT, s2 / DT); };
                f16x8 vq[3];
                vq[0] = vread(0);
                vq[1] = vread(1);
    #pragma unroll
                for (int s2 = 0; s2 < NPV; ++s2) {
                    if (s2 + 2 < NPV) vq[(s2 + 2) % 3] = vread(s2 + 2);
                    const int dt = s2 % DT, ks = s2 / DT;
                    acc[dt] = mfma32x32x16_f16(vq[s2 % 3], pp[ks], acc[dt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // identical in every lane: make the branches below scalar
            const bool keep = __builtin_amdgcn_readfirstlane(kflag) != 0;
            float mn = m2, muse = 0.f, alpha = 1.f;
            if (keep) {
                mn = fmaxf(m2, M);
                muse = (mn == kNegInf) ? 0.f : mn;
                alpha = fast_exp2(m2 - muse);
            }
            float ps0 = 0.f, ps1 = 0.f;
            // Scores of tile kt-1, with the softmax of tile kt (when kept) spread
            // over the MFMA steps; its P reuses the registers the P.V consumed.
            auto body = [&](auto keep_c) {
                constexpr bool KEEP = decltype(keep_c)::value;
                constexpr int NS = 2 * KSTEPS;       // score MFMAs of one tile
                constexpr int EPS = 32 / NS;         // softmax elements per score MFMA
                auto kread = [&](int s2) -> bf16x8 {
                    const int sub = s2 & 1, st = s2 >> 1;
                    const int row = 32 * sub + l32;
                    return *(const bf16x8*)(&kb[row * D + 8 * ((2 * st + hi) ^ (row % QCH))]);
                };
                bf16x8 kq[3];
                kq[0] = kread(0);
                kq[1] = kread(1);
    #pragma unroll
                for (int s2 = 0; s2 < NS; ++s2) {
                    if (s2 + 2 < NS) kq[(s2 + 2) % 3] = kread(s2 + 2);
                    const int sub = s2 & 1, st = s2 >> 1;
                    snext[sub] = mfma32x32x16(kq[s2 % 3], qf[st], st == 0 ? f32x16{} : snext[sub]);
                    if (KEEP) {
    #pragma unroll
                        for (int e2 = 0; e2 < EPS; ++e2) {
                            const int e = s2 * EPS + e2;
                            const int sx = e >> 4, r = e & 15;
                            const float ex = fast_exp2(__builtin_fmaf(scur[sx][r], c2, -muse));
                            if (e2 & 1) ps1 += ex; else ps0 += ex;
                            pp[2 * sx + (r >> 3)][r & 7] = to_f16(ex);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // Issue priority: normal for the score MFMAs and softmax, raised for the
            // rest of the tile (row statistics, vote, barrier, and the next tile's
            // MFMA-only P.V).  When both waves on a SIMD can issue, the one in its
            // serial, latency-bound stretch goes first; the other wave's score
            // MFMAs and softmax fill the gaps.
            __builtin_amdgcn_s_setprio(0);
            if (keep) body(std::true_type{});
            else body(std::false_type{});
            __builtin_amdgcn_s_setprio(1);
            // The kept tile's V copy goes out after the score MFMAs, whose K operand
            // reads it would otherwise meet in LDS, and lands before the next barrier
            // (3% faster at tau = 0, unchanged at tau = 1, against issuing it at the
            // decision).
            if (keep) copy_v(kt, buf);

            pending = false;
            if (keep) {
                const float psum = wave_sum_pair(ps0 + ps1);
                lsum = lsum * alpha + psum;
                m2 = mn;
                thr = (lsum > 0.f) ? m2 + fast_log2(lsum) + theta : kNegInf;
                pend_alpha = alpha;
                pend_buf = buf;
                pending = true;
                if (valid) {
                    const int lim = ik - kt * BK;
                    if (lim >= 0) slots += (lim < BK - 1 ? lim : BK - 1) + 1;
                }
                ++kept_count;
                bitword |= 1u << (kt & 31);
            } else if (STATS) {
                if (has) {
                    const float on = fmaxf(om, M);
                    float osum = 0.f;
    #pragma unroll
                    for (int sub = 0; sub < 2; ++sub)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) osum += fast_exp2(__builtin_fmaf(scur[sub][r], c2, -on));
                    osum = wave_sum_pair(osum);
                    ol = ol * fast_exp2(om - on) + osum;
                    om = on;
                }
            }
            if (want_bits && tid == 0 && ((kt & 31) == 0)) {
                bitrow[kt >> 5] = bitword;
                bitword = 0;
            }
            if (kt >= 1) Mraw = mask_max(kt - 1, snext);
        };

        // Two tiles per iteration, the score buffers swapping roles (one V lane
        // offset instead of one per copy leaves the registers this needs).
        int kt = kt_first;
        for (; kt >= 1; kt -= 2) {
            tile(kt, sA, sB);
            tile(kt - 1, sB, sA);
        }
        if (kt == 0) tile(0, sA, sB);
        if (pending) {
            wait_all_then_barrier();
            if (__ballot(pend_alpha != 1.f) != 0ull) {
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= pend_alpha;
            }
            pv(pend_buf, pp, acc);
        }

        // ---- epilogue: O = acc / l, LSE = (m2 + log2 l) ln 2
        if (valid) {
            const float inv = 1.f / lsum;
            uint16_t* orow = obase + (int64_t)i * p.o_sl;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
    #pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = 32 * dt + 8 * g + 4 * hi;
                    u32x2 pk;
                    pk[0] = float_to_bf16_bits(acc[dt][4 * g + 0] * inv) |
                            (float_to_bf16_bits(acc[dt][4 * g + 1] * inv) << 16);
                    pk[1] = float_to_bf16_bits(acc[dt][4 * g + 2] * inv) |
                            (float_to_bf16_bits(acc[dt][4 * g + 3] * inv) << 16);
                    *(u32x2*)(orow + d0) = pk;
                }
            }
            if (hi == 0) {
                const int64_t ri = rowbase + i;
                const float lz2 = m2 + fast_log2(lsum);
                p.lse[ri] = lz2 * kLn2;
                if (p.kept_slots) p.kept_slots[ri] = slots;
                if (STATS) {
                    float wgt = 0.f;
                    if (ol > 0.f) wgt = 1.f / (1.f + fast_exp2(lz2 - (om + fast_log2(ol))));
                    p.omitted[ri] = wgt;
                }
            }
        }
        if (tid == 0 && p.kept_tiles) p.kept_tiles[(int64_t)bh * p.nQB + qb] = kept_count;
    };

    while (true) {
        if (tid == 0) {
            int u = -1;
            while (qsel < xcd + 8) {
                const int x = qsel & 7;
                const int sl = atomicAdd(p.queue + x, 1);       // slot sl of XCD x's blocks
                const int uu = ((sl / p.chunk) * 8 + x) * p.chunk + sl % p.chunk;
                if (uu < p.nunits) {
                    u = uu;
                    break;
                }
                ++qsel;                                         // queue x is drained
            }
            sUnit = u;
        }
        __syncthreads();
        const int u = sUnit;
        __syncthreads();                         // every wave has read it before the next write
        if (u < 0) break;
        run_unit(u);
    }
}

template <int D, int BQ, int BK>
static hipError_t launch_fwd_t(const FwdParams& p, bool stats, hipStream_t s) {
    constexpr int NT = BQ / 32 * 64;
    if (p.cu_q) {
        const int64_t n = (int64_t)p.Hkv * ((p.max_k + BK - 1) / BK);   // tiles of the longest sequence
        int g = (int)(n < 1 ? 1 : n);
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL((mala_v_to_f16_varlen<D, BK>), dim3(g, p.B), dim3(256), 0, s, p);
    } else {
        const int64_t n = (int64_t)p.B * p.Hkv * (p.Lpad / BK);          // tiles
        int g = (int)(n < 1 ? 1 : n);
        if (g > 16384) g = 16384;
        hipLaunchKernelGGL((mala_v_to_f16<D, BK>), dim3(g), dim3(256), 0, s, p);
    }
    // persistent workgroups: eight waves per CU (two per SIMD, what 256 VGPRs
    // allow), fewer when there are fewer blocks.  The packed layout is a
    // template parameter: the fixed-length kernels see a zero row offset at
    // compile time.
    const int slots = p.ncu * (8 / (NT / 64));
    const int grid = (p.nunits < slots ? (p.nunits + 7) / 8 * 8 : slots);
    const bool vl = p.cu_q != nullptr;
    if (stats && vl)
        hipLaunchKernelGGL((mala_fwd_kernel<D, BQ, BK, true, true>), dim3(grid), dim3(NT), 0, s, p);
    else if (stats)
        hipLaunchKernelGGL((mala_fwd_kernel<D, BQ, BK, true, false>), dim3(grid), dim3(NT), 0, s, p);
    else if (vl)
        hipLaunchKernelGGL((mala_fwd_kernel<D, BQ, BK, false, true>), dim3(grid), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL((mala_fwd_kernel<D, BQ, BK, false, false>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int d, int Bq, int Bk, bool stats, hipStream_t s) {
    if (d == 128 && Bq == 128 && Bk == 64) return launch_fwd_t<128, 128, 64>(p, stats, s);
    if (d == 64 && Bq == 64 && Bk == 64) return launch_fwd_t<64, 64, 64>(p, stats, s);
    return hipErrorInvalidValue;
}

}  // namespace mala
