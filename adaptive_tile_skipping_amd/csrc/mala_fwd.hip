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
// contraction O^T += V^T P^T directly from the score registers.
//   - Q fragments live in registers for the whole loop.
//   - K tiles are double-buffered in LDS; the next tile's global loads are
//     issued before the current tile's MFMAs.
//   - V tiles are fetched only after the keep decision, transposed on the way
//     into LDS (positions inside each 16-key group permuted to match the
//     score-register order) and converted to fp16, exactly for |v| <= 65504.
//   - P.V runs as an fp16 contraction: P in [0, 1] rounded to nearest fp16
//     keeps the relative weight error near 3e-4 (bf16 P would cost ~1e-3 on
//     diffuse rows, as much as the bf16 rounding of O itself).
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {

template <int D, int BQ, int BK, bool STATS>
__global__ __launch_bounds__(BQ / 32 * 64) void mala_fwd_kernel(const FwdParams p) {
    constexpr int NW = BQ / 32;
    constexpr int NT = NW * 64;
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int KROW = D + 8;          // padded LDS row of a K tile (elements)
    constexpr int VROW = BK + 8;         // padded LDS row of a transposed V tile
    constexpr int KCH = D / 8;           // 16-byte chunks per key row
    constexpr int KPASS = BK * KCH / NT;
    constexpr int VPASS = (BK / 4) * KCH / NT;
    static_assert(BK == 64, "tile width");
    static_assert(KPASS * NT == BK * KCH && VPASS * NT == (BK / 4) * KCH, "load split");

    __shared__ __attribute__((aligned(16))) uint16_t sK[2][BK * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t sV[D * VROW];
    __shared__ int sFlag[2][NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int u = xcd_unit(blockIdx.x, p.chunk);
    if (u >= p.nunits) return;
    const int nbh = p.B * p.Hq;
    const int qb = p.nQB - 1 - u / nbh;          // longest blocks first
    const int bh = u % nbh;
    const int b = bh / p.Hq;
    const int h = bh % p.Hq;
    const int kh = h / p.G;
    const int L = p.L;

    const int i0 = qb * BQ;
    const int i = i0 + 32 * w + l32;             // this lane's query row
    const bool valid = i < L;
    const int rend = (i0 + BQ < L) ? i0 + BQ : L;
    const int kt_first = (rend - 1) / BK;

    const uint16_t* kbase = p.k + b * p.k_sb + kh * p.k_sh;
    const uint16_t* vbase = p.v + b * p.v_sb + kh * p.v_sh;

    // ---- Q fragments (B operand: column = query, 8 consecutive d per lane)
    bf16x8 qf[KSTEPS];
    {
        const uint16_t* qrow = p.q + b * p.q_sb + (int64_t)(valid ? i : 0) * p.q_sl + h * p.q_sh;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            u32x4 x = valid ? *(const u32x4*)(qrow + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            qf[st] = __builtin_bit_cast(bf16x8, x);
        }
    }

    u32x4 kreg[KPASS];
    auto load_k = [&](int kt) {
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            const int idx = tid + ps * NT;
            const int r = idx / KCH, c = idx % KCH;
            const int j = kt * BK + r;
            kreg[ps] = (j < L) ? *(const u32x4*)(kbase + (int64_t)j * p.k_sl + 8 * c) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_k = [&](int buf) {
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            const int idx = tid + ps * NT;
            const int r = idx / KCH, c = idx % KCH;
            *(u32x4*)(&sK[buf][r * KROW + 8 * c]) = kreg[ps];
        }
    };
    u32x4 vreg[VPASS][4];
    auto load_v = [&](int kt) {
#pragma unroll
        for (int ps = 0; ps < VPASS; ++ps) {
            const int idx = tid + ps * NT;
            const int kq = idx % (BK / 4), dc = idx / (BK / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kt * BK + 4 * kq + r;
                vreg[ps][r] = (j < L) ? *(const u32x4*)(vbase + (int64_t)j * p.v_sl + 8 * dc) : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_vt = [&]() {
#pragma unroll
        for (int ps = 0; ps < VPASS; ++ps) {
            const int idx = tid + ps * NT;
            const int kq = idx % (BK / 4), dc = idx / (BK / 4);
            const int pos = 16 * (kq >> 2) + vt_pos16(4 * (kq & 3));
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t a0 = vreg[ps][0][m], a1 = vreg[ps][1][m];
                const uint32_t a2 = vreg[ps][2][m], a3 = vreg[ps][3][m];
                u32x2 lo = {pack2_f16_from_f32bits(a0 << 16, a1 << 16), pack2_f16_from_f32bits(a2 << 16, a3 << 16)};
                u32x2 hv = {pack2_f16_from_f32bits(a0 & 0xFFFF0000u, a1 & 0xFFFF0000u),
                            pack2_f16_from_f32bits(a2 & 0xFFFF0000u, a3 & 0xFFFF0000u)};
                *(u32x2*)(&sV[(8 * dc + 2 * m) * VROW + pos]) = lo;
                *(u32x2*)(&sV[(8 * dc + 2 * m + 1) * VROW + pos]) = hv;
            }
        }
    };

    // ---- per-row state (this lane's query; lanes l and l^32 hold identical copies)
    float m2 = kNegInf;          // running max of retained base-2 scores
    float lsum = 0.f;            // retained sum, shifted by m2
    float thr = kNegInf;         // cached keep threshold m2 + log2(lsum) + theta
    const float theta = p.log2_tau - fast_log2((float)(i + 1));
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

    load_k(kt_first);
    store_k(0);
    __syncthreads();

    for (int it = 0; it <= kt_first; ++it) {
        const int kt = kt_first - it;
        const int buf = it & 1;
        if (kt > 0) load_k(kt - 1);

        // ---- score discovery: S^T = K Q^T for the two 32-key subtiles
        f32x16 s[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            s[sub] = f32x16{};
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                const bf16x8 a = *(const bf16x8*)(&sK[buf][(32 * sub + l32) * KROW + 16 * st + 8 * hi]);
                s[sub] = mfma32x32x16(a, qf[st], s[sub]);
            }
        }
        // scale to base 2 and mask illegal keys (j > i, or invalid row)
        const int lim = valid ? (i - kt * BK) : -1;   // last legal key offset in the tile
        float M = kNegInf;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int jj = 32 * sub + 8 * (r >> 2) + 4 * hi + (r & 3);
                float x = s[sub][r] * p.scale_log2;
                x = (jj <= lim) ? x : kNegInf;
                s[sub][r] = x;
                M = fmaxf(M, x);
            }
        }
        M = wave_max_pair(M);

        // ---- keep decision
        const bool has = M > kNegInf;
        const bool vote = has && (lsum == 0.f || M >= thr);
        const bool wave_any = __ballot(vote) != 0ull;
        if (lane == 0) sFlag[buf][w] = wave_any ? 1 : 0;
        if (kt > 0) store_k(buf ^ 1);
        __syncthreads();
        bool keep = false;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) keep |= (sFlag[buf][ww] != 0);

        if (keep) {
            load_v(kt);
            // online-softmax update of this row
            const float mn = fmaxf(m2, M);
            const float muse = (mn == kNegInf) ? 0.f : mn;
            const float alpha = fast_exp2(m2 - muse);
            float psum = 0.f;
            f16x8 pb[4];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(s[sub][r] - muse);
                    psum += e;
                    pb[2 * sub + (r >> 3)][r & 7] = to_f16(e);
                }
            }
            psum = wave_sum_pair(psum);
            lsum = lsum * alpha + psum;
            m2 = mn;
            thr = (lsum > 0.f) ? m2 + fast_log2(lsum) + theta : kNegInf;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
            if (lim >= 0) slots += (lim < BK - 1 ? lim : BK - 1) + 1;
            store_vt();
            __syncthreads();
            // O^T += V^T P^T
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const f16x8 a = *(const f16x8*)(&sV[(32 * dt + l32) * VROW + 16 * ks + 8 * hi]);
                    acc[dt] = mfma32x32x16_f16(a, pb[ks], acc[dt]);
                }
            }
            ++kept_count;
            bitword |= 1u << (kt & 31);
        } else if (STATS) {
            if (has) {
                const float mn = fmaxf(om, M);
                float osum = 0.f;
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int r = 0; r < 16; ++r) osum += fast_exp2(s[sub][r] - mn);
                osum = wave_sum_pair(osum);
                ol = ol * fast_exp2(om - mn) + osum;
                om = mn;
            }
        }
        if (want_bits && tid == 0 && ((kt & 31) == 0)) {
            bitrow[kt >> 5] = bitword;
            bitword = 0;
        }
    }

    // ---- epilogue: O = acc / l, LSE = (m2 + log2 l) ln 2
    if (valid) {
        const float inv = 1.f / lsum;
        uint16_t* orow = p.o + b * p.o_sb + (int64_t)i * p.o_sl + h * p.o_sh;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * dt + 8 * g + 4 * hi;
                u32x2 pk;
                pk[0] = float_to_bf16_bits(acc[dt][4 * g + 0] * inv) | (float_to_bf16_bits(acc[dt][4 * g + 1] * inv) << 16);
                pk[1] = float_to_bf16_bits(acc[dt][4 * g + 2] * inv) | (float_to_bf16_bits(acc[dt][4 * g + 3] * inv) << 16);
                *(u32x2*)(orow + d0) = pk;
            }
        }
        if (hi == 0) {
            const int64_t ri = (int64_t)bh * L + i;
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
}

template <int D, int BQ, int BK>
static hipError_t launch_fwd_t(const FwdParams& p, bool stats, hipStream_t s) {
    constexpr int NT = BQ / 32 * 64;
    const int per = 8 * p.chunk;
    const int grid = (p.nunits + per - 1) / per * per;
    if (stats)
        hipLaunchKernelGGL((mala_fwd_kernel<D, BQ, BK, true>), dim3(grid), dim3(NT), 0, s, p);
    else
        hipLaunchKernelGGL((mala_fwd_kernel<D, BQ, BK, false>), dim3(grid), dim3(NT), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int d, int Bq, int Bk, bool stats, hipStream_t s) {
    if (d == 128 && Bq == 128 && Bk == 64) return launch_fwd_t<128, 128, 64>(p, stats, s);
    if (d == 64 && Bq == 64 && Bk == 64) return launch_fwd_t<64, 64, 64>(p, stats, s);
    return hipErrorInvalidValue;
}

}  // namespace mala
