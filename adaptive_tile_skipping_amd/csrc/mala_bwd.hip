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
//   mala_bwd_pre    D_i and LSE_i in base 2 per row, zeroed tile bits and
//                   statistics.
//   mala_bwd_scan   the decision pass (tau > 0): one workgroup per (batch, q
//                   head, 256-query slab), 4 waves of 64 queries.  Q and each
//                   row's threshold stay in registers; key tiles stream from
//                   the slab's diagonal to key 0 through a triple-buffered LDS
//                   tile.  The score accumulator starts at minus the row's
//                   threshold, so a tile is kept iff the masked maximum of the
//                   accumulator is >= 0.  A kept tile sets its bit in the key
//                   tile's word row (q head, query block) and in the query
//                   block's word row (key tile); nothing else is written, so
//                   skipped tiles cost only the score MFMAs.
//   mala_bwd_kernel the dK/dV pass: one workgroup per (batch, KV head, key
//                   tile of 64 keys), 4 waves, visiting only the kept (q head,
//                   query block) steps of its key tile (all legal steps when
//                   tau = 0).  K and V fragments stay in registers; each step's
//                   Q and dO blocks stream through double-buffered LDS tiles and
//                   S = Q K^T, dP = dO V^T are recomputed.  Wave w owns keys
//                   32(w&1).. and half (w>>1) of the block's queries.  S is laid
//                   out with one key per lane and the block's queries in
//                   registers, so P^T and dS^T feed the dV and dK contractions
//                   straight from registers, with dO^T and Q^T from transposing
//                   LDS reads; dK/dV accumulate in registers over steps.  A
//                   wave takes its 32-query subtiles one at a time through
//                   scores, softmax and contractions.  At tau = 0, when there
//                   are enough units to fill the device, a workgroup owns two
//                   adjacent key tiles instead: wave w holds keys 32 w .. of
//                   the 128 and takes all four query subtiles of the block, so
//                   each streamed block serves twice the keys; those units
//                   start longest first.  The causal mask is applied only on
//                   steps that cross the diagonal or the sequence end.
//   mala_bwd_dq     the dQ pass: one workgroup per (batch, q head, query
//                   block), waves of 32 queries, visiting the block's kept key
//                   tiles (all legal tiles when tau = 0) with K and V tiles
//                   double-buffered in LDS: S^T = K Q^T and dP^T = V dO^T, then
//                   dQ^T += K^T dS^T with K^T from LDS transposing reads.  dQ is
//                   accumulated in registers and written once: no atomics.
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {

namespace {
constexpr int BK = 64;
constexpr int PRE_ROWS = 64;

}  // namespace

// One sequence as the kernels see it: Lq queries that are the last Lq of its
// Lk keys (Lq = Lk = L for the fixed-length layout), so query row i sees keys
// j <= off + i and has L_i = off + i + 1.  Pointers address row 0 of the
// sequence (head 0); lse / kept_slots entries of (h, i) sit at
// lse0 + h lse_hs + i, the row terms at row0 + h row_hs + i.  A packed
// sequence whose lengths are inconsistent with the call's totals and maxima
// reads as empty (Lq = Lk = 0) and is skipped.
struct SeqView {
    int Lq, Lk, off;
    const uint16_t *q, *k, *v, *o, *dout;
    uint16_t *dq, *dk, *dv;
    int64_t lse0, lse_hs, row0, row_hs;
};
template <int BQ, bool VARLEN>
__device__ __forceinline__ SeqView seq_view(const BwdParams& p, int b) {
    SeqView s;
    if constexpr (VARLEN) {
        const int q0 = p.cu_q[b], q1 = p.cu_q[b + 1], k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
        const bool ok = q0 >= 0 && k0 >= 0 && q1 <= p.total_q && k1 <= p.total_k && q1 - q0 >= 0 &&
                        k1 - k0 >= q1 - q0 && q1 - q0 <= p.max_q && k1 - k0 <= p.max_k;
        s.Lq = ok ? q1 - q0 : 0;
        s.Lk = ok ? k1 - k0 : 0;
        s.q = p.q + (int64_t)q0 * p.q_sl;
        s.o = p.o + (int64_t)q0 * p.o_sl;
        s.dout = p.dout + (int64_t)q0 * p.do_sl;
        s.dq = p.dq + (int64_t)q0 * p.dq_sl;
        s.k = p.k + (int64_t)k0 * p.k_sl;
        s.v = p.v + (int64_t)k0 * p.v_sl;
        s.dk = p.dk + (int64_t)k0 * p.dk_sl;
        s.dv = p.dv + (int64_t)k0 * p.dv_sl;
        s.lse0 = q0;
        s.lse_hs = p.total_q;
        s.row0 = (int64_t)q0 + (int64_t)b * BQ;
        s.row_hs = p.Rq;
    } else {
        s.Lq = s.Lk = p.L;
        s.q = p.q + b * p.q_sb;
        s.o = p.o + b * p.o_sb;
        s.dout = p.dout + b * p.do_sb;
        s.dq = p.dq + b * p.dq_sb;
        s.k = p.k + b * p.k_sb;
        s.v = p.v + b * p.v_sb;
        s.dk = p.dk + b * p.dk_sb;
        s.dv = p.dv + b * p.dv_sb;
        s.lse0 = (int64_t)b * p.Hq * p.L;
        s.lse_hs = p.L;
        s.row0 = (int64_t)b * p.Hq * p.Lpad;
        s.row_hs = p.Lpad;
    }
    s.off = s.Lk - s.Lq;
    return s;
}

template <int D, int BQ, bool VARLEN>
__global__ __launch_bounds__(256) void mala_bwd_pre(const BwdParams p) {
    const int tid = threadIdx.x;
    const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int r0 = rb * PRE_ROWS;
    const SeqView sv = seq_view<BQ, VARLEN>(p, b);
    const int L = sv.Lq;
    const int Lrows = (L + BQ - 1) / BQ * BQ;     // the sequence's padded row-term rows
    const int64_t bh = (int64_t)b * p.Hq + h;
    // D_i = dO_i . O_i and LSE in base 2 (4 threads per row; 0 past L)
    {
        const int r = tid >> 2, part = tid & 3;
        const int i = r0 + r;
        float acc = 0.f;
        if (i < L) {
            const uint16_t* orow = sv.o + (int64_t)i * p.o_sl + h * p.o_sh;
            const uint16_t* grow = sv.dout + (int64_t)i * p.do_sl + h * p.do_sh;
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
        if (part == 0 && i < Lrows) {
            const int64_t ri = sv.row0 + h * sv.row_hs + i;
            const int64_t li = sv.lse0 + h * sv.lse_hs + i;
            p.rowd[ri] = (i < L) ? acc : 0.f;
            p.rowc[ri] = (i < L) ? p.lse[li] * kLog2e : 0.f;
            if (p.kept_slots && i < L) p.kept_slots[li] = 0;
        }
    }
    // zero the kept-tile bits (the scan only sets bits)
    if (p.log2_tau != kNegInf) {
        const int64_t nblk = (int64_t)gridDim.x * gridDim.y * gridDim.z;
        const int64_t fb = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        const int64_t nw = (int64_t)p.B * p.Hkv * p.nKT * p.nwT;
        for (int64_t idx = fb * 256 + tid; idx < nw; idx += nblk * 256) p.tbits[idx] = 0u;
        const int64_t nq = (int64_t)p.B * p.Hq * p.nQB * p.nwords;
        for (int64_t idx = fb * 256 + tid; idx < nq; idx += nblk * 256) p.qbits[idx] = 0u;
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
}

// Decision pass of the backward (tau > 0).  See the file comment.
template <int D, int BQ, bool VARLEN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mala_bwd_scan(
    const BwdParams p) {
    constexpr int KSTEPS = D / 16;
    constexpr int QCH = D / 8;             // 16-byte chunks per row
    constexpr int KINST = BK * QCH / 256;  // global->LDS copies per lane per key tile
    constexpr int NB = 4;                  // two pairs of key tiles: the current pair and the next
    static_assert(KINST * 256 == BK * QCH, "shape");
    // key tiles [NB][BK][D] bf16, chunk c of row r stored at chunk c ^ (r % QCH)
    __shared__ __attribute__((aligned(16))) uint16_t sK[NB][BK * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int u = xcd_unit(blockIdx.x, p.chunk_scan);
    if (u >= p.nunits_scan) return;
    const int BH = p.B * p.Hq;
    const int slab = p.nslab - 1 - u / BH;   // longest slabs first
    const int b = (u % BH) / p.Hq;
    const int h = (u % BH) % p.Hq;
    const int kh = h / p.G;
    const SeqView sv = seq_view<BQ, VARLEN>(p, b);
    const int L = sv.Lq, Lk = sv.Lk, off = sv.off;
    const int R0 = slab * 256;
    if (R0 >= L) return;                     // past the sequence's queries
    const int rw0 = R0 + 64 * w;             // the wave's 64 queries
    const int last = (R0 + 255 < L - 1) ? R0 + 255 : L - 1;
    const int kt_hi = (off + last) / BK;
    const bool live = rw0 < L;
    // the wave's last key tile with a legal entry, and the key offset of its
    // first row's last legal key: tiles ending past it need the causal mask
    const int kt_w = live ? (off + ((rw0 + 63 < L - 1) ? rw0 + 63 : L - 1)) / BK : -1;
    const int jdiag = off + rw0;
    const float c2 = p.scale_log2;
    const int64_t bh = (int64_t)b * p.Hq + h;

    // ---- Q fragments (A operands: row = query, 8 consecutive d) and the seeds:
    // minus each row's threshold on raw scores, -inf past L
    bf16x8 qa[2][KSTEPS];
    f32x16 seed[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int i = rw0 + 32 * t + l32;
        const bool ok = i < L;
        const uint16_t* qr = sv.q + (int64_t)(ok ? i : 0) * p.q_sl + h * p.q_sh;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            const u32x4 x = ok ? *(const u32x4*)(qr + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            qa[t][st] = __builtin_bit_cast(bf16x8, x);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ir = rw0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
            seed[t][r] = (ir < L) ? -(p.lse[sv.lse0 + h * sv.lse_hs + ir] * kLog2e +
                                      (p.log2_tau - fast_log2((float)(off + ir + 1)))) / c2
                                  : kNegInf;
        }
    }

    // ---- key tile copies through a buffer resource ending at key L-1
    uint32_t koff[KINST];
#pragma unroll
    for (int n = 0; n < KINST; ++n) {
        const int sl = (n * 4 + w) * 64 + lane;
        const int r = sl / QCH, pc = sl % QCH;
        koff[n] = (uint32_t)((r * p.k_sl + 8 * (pc ^ (r % QCH))) * 2);
    }
    const uint16_t* kbase = sv.k + kh * p.k_sh;
    auto copy_tile = [&](int kt, int buf) {
        const int j0 = kt * BK;
        const int nrow = (Lk - j0 < BK) ? Lk - j0 : BK;
        const __amdgpu_buffer_rsrc_t rk =
            make_rsrc(kbase + (int64_t)j0 * p.k_sl, (uint32_t)(((nrow - 1) * p.k_sl + D) * 2));
        unsigned char* dst = reinterpret_cast<unsigned char*>(sK[buf]);
#pragma unroll
        for (int n = 0; n < KINST; ++n) buffer16_to_lds(rk, koff[n], dst + (n * 4 + w) * 64 * 16);
    };

    // Key tiles are processed in pairs, one barrier per pair: pair q holds tiles
    // kt_hi - 2q and kt_hi - 2q - 1 in slots 2(q & 1) and 2(q & 1) + 1.
    const int nt = kt_hi + 1;
    const int npair = (nt + 1) / 2;
    auto copy_pair = [&](int q) {
        const int kt = kt_hi - 2 * q;
        copy_tile(kt, 2 * (q & 1));
        if (kt >= 1) copy_tile(kt - 1, 2 * (q & 1) + 1);
    };
    copy_pair(0);

    uint32_t* bitrow = p.tbits + (int64_t)(b * p.Hkv + kh) * p.nKT * p.nwT;
    const int bit = (h % p.G) * p.nQB + rw0 / BQ;
    uint32_t* qrow = p.qbits + (bh * p.nQB + rw0 / BQ) * p.nwords;

    for (int q = 0; q < npair; ++q) {
        // pair q has landed, and every wave is done with pair q - 1, whose
        // slots take pair q + 1
        wait_all_then_barrier();
        if (q + 1 < npair) copy_pair(q + 1);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
        const int kt = kt_hi - 2 * q - half;
        const int buf = 2 * (q & 1) + half;
        if (kt >= 0 && live && kt <= kt_w) {
            const uint16_t* sKb = sK[buf];
            f32x16 acc[2][2];
            // K fragments are read one k-step ahead (a two-slot ring); a
            // scheduling barrier closes every step to keep that order
            auto kread = [&](int st, int uu) -> bf16x8 {
                const int row = 32 * uu + l32;
                return *(const bf16x8*)(&sKb[row * D + 8 * ((2 * st + hi) ^ (row % QCH))]);
            };
            bf16x8 kb[2][2];
            kb[0][0] = kread(0, 0);
            kb[0][1] = kread(0, 1);
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                if (st + 1 < KSTEPS) {
                    kb[(st + 1) & 1][0] = kread(st + 1, 0);
                    kb[(st + 1) & 1][1] = kread(st + 1, 1);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int uu = 0; uu < 2; ++uu)
                        acc[t][uu] = mfma32x32x16(qa[t][st], kb[st & 1][uu], st == 0 ? seed[t] : acc[t][uu]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // C[i = query][j = key]: lane = key 32uu + l32, register r = query
            // 32t + 8(r/4) + 4hi + r%4.  Keep iff a legal entry is >= 0.
            float mx = kNegInf;
            if (kt * BK + BK - 1 > jdiag) {
                // key kt BK + 32uu + l32 is legal for query rw0 + iq iff it is <= off + rw0 + iq
                const int kk = kt * BK + l32 - jdiag;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int iq = 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
                            mx = fmaxf(mx, (kk + 32 * uu <= iq) ? acc[t][uu][r] : kNegInf);
                        }
            } else {
                // four independent chains, then combined
                float m4[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    m4[c] = acc[c >> 1][c & 1][0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) m4[c] = fmaxf(m4[c], acc[c >> 1][c & 1][r]);
                }
                mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            }
            if (__ballot(mx >= 0.f) != 0ull && lane == 0) {
                atomicOr(bitrow + (int64_t)kt * p.nwT + (bit >> 5), 1u << (bit & 31));
                atomicOr(qrow + (kt >> 5), 1u << (kt & 31));
            }
        }
        }
    }
}

// Enumerates the steps of one key tile as hl * nQB + qb (hl = q head within
// the KV group).  Dense (tau = 0): every q head, query blocks newest first down
// to the block holding the tile.  Sparse: the set bits of the tile's word row
// in increasing order, read 64 words (one per lane) at a time.  All state but
// `my` is wave-uniform.
struct StepCursor {
    const uint32_t* words;
    int nw, wb, wi;
    uint32_t my, cur;
    uint64_t mask;
    bool dense;
    int hl, qb, qb_lo, qb_hi, nQB, G;

    // dense: blocks qb_hi down to qb_lo of every q head (none if qb_hi < qb_lo);
    // nQB is the stride of the step index
    __device__ void init(bool dense_, const uint32_t* words_, int nw_, int qb_lo_, int qb_hi_, int nQB_, int G_) {
        dense = dense_; words = words_; nw = nw_;
        wb = -64; wi = -65; my = 0u; cur = 0u; mask = 0ull;
        hl = 0; qb = qb_hi_; qb_lo = qb_lo_; qb_hi = qb_hi_; nQB = nQB_; G = G_;
    }
    __device__ int next(int lane) {
        if (dense) {
            if (hl >= G || qb_hi < qb_lo) return -1;
            const int idx = hl * nQB + qb;
            if (--qb < qb_lo) { qb = qb_hi; ++hl; }
            return idx;
        }
        for (;;) {
            if (cur) {
                const int bpos = __builtin_ctz(cur);
                cur &= cur - 1u;
                return wi * 32 + bpos;
            }
            const int off = wi - wb;   // -1 .. 63
            const uint64_t m = (off >= 63) ? 0ull : (mask & (~0ull << (off + 1)));
            if (m == 0ull) {
                wb += 64;
                if (wb >= nw) return -1;
                my = (wb + lane < nw) ? words[wb + lane] : 0u;
                mask = __ballot(my != 0u);
                wi = wb - 1;
                continue;
            }
            const int o = __builtin_ctzll(m);
            wi = wb + o;
            cur = (uint32_t)__builtin_amdgcn_readlane((int)my, o);
        }
    }
};

// LDS row swizzle for tiles read both row-wise (16-byte MFMA operand reads)
// and transposed (ds_read_b64_tr_b16): 16-byte chunk c of row r lives at chunk
// c ^ kswz(r).  The LDS has 64 four-byte banks, one 256-byte row of a d = 128
// tile.  A 16-byte read serves 16 lanes per pass: kswz permutes 0..15 over 16
// consecutive rows, so those lanes (16 rows, one logical chunk) hit 16
// different chunks.  An 8-byte transposing read serves 32 lanes per pass: four
// consecutive rows, 64 bytes (four chunks) each; kswz puts each of the four
// rows in a different group of four chunks (4 (r & 3) + ...), so the pass
// covers all 64 banks once.  For d = 64 (8 chunks, two rows per bank line) the
// earlier form is kept: the four rows of a transposing read get four
// different chunk pairs.
template <int QCH>
__device__ __forceinline__ int kswz(int r) {
    if constexpr (QCH == 16) return 4 * (r & 3) + ((r >> 2) & 3);
    else return (2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1)) % QCH;
}

template <int D, int BQ, bool VARLEN, bool WIDE>
__global__ __launch_bounds__(256) void mala_bwd_kernel(const BwdParams p) {
    // WIDE (tau = 0 only): a workgroup owns two key tiles, wave w keys 32 w ..
    // 32 w + 31 of them, and takes every query subtile of the block, so each
    // streamed Q / dO block serves twice the keys.
    constexpr int KT_PER = WIDE ? 2 : 1;       // key tiles per workgroup
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int NQS = BQ / 32;         // query subtiles of the block
    constexpr int WSUB = NQS / 2;        // query subtiles per wave (one key tile per unit)
    constexpr int NSUB = WIDE ? NQS : WSUB;   // query subtiles a wave visits per step
    constexpr int QCH = D / 8;           // 16-byte chunks per row
    constexpr int QSLOTS = BQ * QCH;     // 16-byte chunks per block (each of Q, dO)
    constexpr int QINST = QSLOTS / 256;  // global->LDS copies per lane per block and tensor
    constexpr int BLK = BQ * D;          // elements of one block
    constexpr int QBYTES = 2 * 2 * BLK * 2;               // [buf][Q | dO] blocks
    constexpr int RBYTES = 2 * 2 * DT * 16 * 64 * 4;     // epilogue reduction
    constexpr int UBYTES = QBYTES > RBYTES ? QBYTES : RBYTES;
    static_assert(QINST * 256 == QSLOTS && WSUB >= 1, "shape");

    // [buf][Q | dO][BQ][D] bf16, 16-byte chunk c of row r stored at chunk c ^ kswz(r)
    __shared__ __attribute__((aligned(16))) unsigned char sU[UBYTES];
    // [buf][lse2 | D][query]
    __shared__ __attribute__((aligned(16))) float sRow[2][2][BQ];
    uint16_t* sQD = reinterpret_cast<uint16_t*>(sU);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int kw = WIDE ? w : (w & 1);
    const int qh0 = WIDE ? 0 : (w >> 1);
    const int SUB0 = WIDE ? 0 : WSUB * qh0;   // the wave's first query subtile

    // Work units: KT_PER adjacent key tiles of one (batch, KV head); `chunk`
    // consecutive units run on one XCD.
    const int nKTu = (p.nKT + KT_PER - 1) / KT_PER;   // units per (batch, KV head)
    const int nbk = p.B * p.Hkv;
    const int u = xcd_unit(blockIdx.x, p.chunk);
    int bk, ku;
    if (p.log2_tau == kNegInf) {
        // tau = 0: a unit's length is the number of query blocks that see it.
        // Chunks of adjacent units go in increasing key order across every
        // (batch, KV head), so the longest units start first.
        const int ch = u / p.chunk;
        if (ch >= (nKTu + p.chunk - 1) / p.chunk * nbk) return;
        bk = ch % nbk;
        ku = (ch / nbk) * p.chunk + u % p.chunk;
    } else {
        // tau > 0: (batch, KV head) major, key units in increasing order, so the
        // units running together mostly share one KV head's Q / dO blocks in L2
        if (u >= nbk * nKTu) return;
        bk = u / nKTu;
        ku = u % nKTu;
    }
    if (ku >= nKTu) return;
    const int kt = ku * KT_PER;             // first key tile of the unit
    const int b = bk / p.Hkv;
    const int kh = bk % p.Hkv;
    const SeqView sv = seq_view<BQ, VARLEN>(p, b);
    const int L = sv.Lq, Lk = sv.Lk, off = sv.off;
    const int j0 = kt * BK;
    if (j0 >= Lk) return;                   // past the sequence's keys
    const int G = p.G;
    const float c2 = p.scale_log2;

    // ---- resident K and V fragments (B operands: column = key, 8 consecutive d)
    const int jme = j0 + 32 * kw + l32;
    bf16x8 kf[KSTEPS], vf[KSTEPS];
    {
        const bool ok = jme < Lk;
        const uint16_t* kr = sv.k + (int64_t)(ok ? jme : 0) * p.k_sl + kh * p.k_sh;
        const uint16_t* vr = sv.v + (int64_t)(ok ? jme : 0) * p.v_sl + kh * p.v_sh;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            const u32x4 a = ok ? *(const u32x4*)(kr + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            const u32x4 c = ok ? *(const u32x4*)(vr + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            kf[st] = __builtin_bit_cast(bf16x8, a);
            vf[st] = __builtin_bit_cast(bf16x8, c);
        }
    }
    f32x16 dv[DT], dk[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { dv[dt] = f32x16{}; dk[dt] = f32x16{}; }

    // query blocks that can see the tile: from the one holding row j0 - off
    const int qb_lo = (j0 - off > 0 ? j0 - off : 0) / BQ;
    const int qb_hi = (L + BQ - 1) / BQ - 1;
    const bool dense = WIDE || p.log2_tau == kNegInf;   // tau = 0: every legal step is kept
    const uint32_t* trow = p.tbits + ((int64_t)(b * p.Hkv + kh) * p.nKT + kt) * p.nwT;

    // Per-lane byte offsets of this lane's 16-byte chunks inside a Q / dO block
    uint32_t qoff[QINST], goff[QINST];
#pragma unroll
    for (int n = 0; n < QINST; ++n) {
        const int sl = (n * 4 + w) * 64 + lane;
        const int r = sl / QCH, pc = sl % QCH;
        const int c = pc ^ kswz<QCH>(r);
        qoff[n] = (uint32_t)((r * p.q_sl + 8 * c) * 2);
        goff[n] = (uint32_t)((r * p.do_sl + 8 * c) * 2);
    }
    // issue the copies of step `idx` (q head kh*G + idx / nQB, query block
    // idx % nQB): its row terms, Q block and dO block, into buffer `buf`
    auto fetch = [&](int idx, int buf) {
        const int f_h = kh * G + idx / p.nQB, f_qb = idx % p.nQB;
        const int row0 = f_qb * BQ;
        // the blocks' rows through buffer resources ending at row L-1, so the
        // rows past L read as zero without per-lane clamps
        const int nrow = (L - row0 < BQ) ? L - row0 : BQ;
        const uint16_t* qblk = sv.q + (int64_t)row0 * p.q_sl + f_h * p.q_sh;
        const uint16_t* gblk = sv.dout + (int64_t)row0 * p.do_sl + f_h * p.do_sh;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(qblk, (uint32_t)(((nrow - 1) * p.q_sl + D) * 2));
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(gblk, (uint32_t)(((nrow - 1) * p.do_sl + D) * 2));
        unsigned char* dq_ = sU + buf * (2 * BLK * 2);
        unsigned char* dg_ = dq_ + BLK * 2;
#pragma unroll
        for (int n = 0; n < QINST; ++n) {
            buffer16_to_lds(rq, qoff[n], dq_ + (n * 4 + w) * 64 * 16);
            buffer16_to_lds(rg, goff[n], dg_ + (n * 4 + w) * 64 * 16);
        }
        // row terms: waves 0..1 copy lse2 / D (BQ floats each); last, so the
        // resources above are not held across this lane-divergent branch
        if (w < 2 && lane * 4 < BQ) {
            const float* src = (w == 0 ? p.rowc : p.rowd) + sv.row0 + f_h * sv.row_hs + row0;
            load16_to_lds(src + 4 * lane, &sRow[buf][w][0]);
        }
    };
    // every copy of the step fetched last may stay in flight
    auto wait_prev = [&](bool more) {
        if (!more) wait_vmcnt<0>();
        else if (w < 2) wait_vmcnt<2 * QINST + 1>();
        else wait_vmcnt<2 * QINST>();
    };

    const int j16 = lane & 15;
    const int dsel = 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);
    // B operand of dV / dK: 8 queries (in the score registers' order) of one d,
    // by transposing reads of a row-major block
    auto tread = [&](const uint16_t* blk, int qrow0, int dt) -> bf16x8 {
        u32x2 half2x[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int row = qrow0 + 8 * rd + 4 * hi + (j16 >> 2);
            const int col = 32 * dt + dsel;
            const int phys = ((col >> 3) ^ kswz<QCH>(row)) * 8 + (col & 7);
            half2x[rd] = lds_read_tr16(blk + row * D + phys);
        }
        const u32x4 w4 = {half2x[0][0], half2x[0][1], half2x[1][0], half2x[1][1]};
        return __builtin_bit_cast(bf16x8, w4);
    };

    StepCursor cc;
    cc.init(dense, trow, p.nwT, qb_lo, qb_hi, p.nQB, G);
    // The step index is the same in every lane; read as uniform, the copies'
    // buffer resources stay scalar (no per-copy waterfall loop).
    auto next_step = [&]() -> int { return __builtin_amdgcn_readfirstlane(cc.next(lane)); };
    int cur = next_step(), nxt = -1;
    if (cur >= 0) {
        fetch(cur, 0);
        nxt = next_step();
        if (nxt >= 0) fetch(nxt, 1);
        wait_prev(nxt >= 0);
        __syncthreads();
    }

    for (int s = 0; cur >= 0; ++s) {
        const int buf = s & 1;
        const int h = kh * G + cur / p.nQB;
        const int qb = cur % p.nQB;
        const uint16_t* sQb = sQD + buf * 2 * BLK;
        const uint16_t* sGb = sQb + BLK;
        const int64_t bh = (int64_t)b * p.Hq + h;
        // every row of the block sees every key of the unit: no causal or
        // length mask on this step
        const bool full = (j0 + BK * KT_PER - 1 <= off + qb * BQ) && (qb * BQ + BQ <= L);
        // The wave's 32-query subtiles go one at a time through scores,
        // softmax and the dV / dK contractions (a whole half at once needs
        // more registers than the allocator handles well).  The scheduling
        // groups keep the LDS operand reads several MFMAs ahead of their use.
#pragma unroll
        for (int g = 0; g < NSUB; ++g) {
            const int qs = SUB0 + g;               // query subtile
            // ---- S = Q K^T and dP = dO V^T for the subtile x the wave's 32 keys
            f32x16 sc = f32x16{}, dp = f32x16{};
            {
                const int row = 32 * qs + l32;
#pragma unroll
                for (int st = 0; st < KSTEPS; ++st) {
                    const int pc = (2 * st + hi) ^ kswz<QCH>(row);
                    const bf16x8 a = *(const bf16x8*)(&sQb[row * D + 8 * pc]);
                    const bf16x8 gg = *(const bf16x8*)(&sGb[row * D + 8 * pc]);
                    sc = mfma32x32x16(a, kf[st], sc);
                    dp = mfma32x32x16(gg, vf[st], dp);
                }
            }
            {   // one operand read per MFMA, PRE MFMAs ahead
                constexpr int NM = 2 * KSTEPS, PRE = NM < 6 ? NM : 6;
                __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
                for (int i = 0; i < NM - PRE; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
            }
            // ---- P, dS; A operands (key rows x 8 permuted query positions) for dV, dK
            bf16x8 pa[2], da[2];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int ql = 32 * qs + 8 * g4 + 4 * hi;
                const f32x4 lv = *(const f32x4*)(&sRow[buf][0][ql]);
                const f32x4 dd = *(const f32x4*)(&sRow[buf][1][ql]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g4 + e;
                    const float pr = fast_exp2(__builtin_fmaf(sc[r], c2, -lv[e]));
                    const float ds = pr * (dp[r] - dd[e]);
                    pa[r >> 3][r & 7] = to_bf16(pr);
                    da[r >> 3][r & 7] = to_bf16(ds);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (!full) {
                // a diagonal or ragged step: P and dS of the pairs that the
                // causal order or the sequence end rules out become 0
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    u32x4 pw = __builtin_bit_cast(u32x4, pa[hf]);
                    u32x4 dw = __builtin_bit_cast(u32x4, da[hf]);
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2) {
                        uint32_t m = 0;
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int r = 8 * hf + 2 * k2 + hh;
                            const int ig = qb * BQ + 32 * qs + 8 * (r >> 2) + 4 * hi + (r & 3);
                            if ((jme <= off + ig) && (ig < L)) m |= 0xFFFFu << (16 * hh);
                        }
                        pw[k2] &= m;
                        dw[k2] &= m;
                    }
                    pa[hf] = __builtin_bit_cast(bf16x8, pw);
                    da[hf] = __builtin_bit_cast(bf16x8, dw);
                }
            }
            // ---- dV += P^T dO, dK += dS^T Q  (B operands by transposing reads)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int qrow0 = 32 * qs + 16 * ks;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    dv[dt] = mfma32x32x16(pa[ks], tread(sGb, qrow0, dt), dv[dt]);
                    dk[dt] = mfma32x32x16(da[ks], tread(sQb, qrow0, dt), dk[dt]);
                }
            }
            {   // two transposing reads per MFMA, PRE MFMAs ahead
                constexpr int NM = 2 * 2 * DT, PRE = 4;
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * PRE, 0);
#pragma unroll
                for (int i = 0; i < NM - PRE; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- statistics of the backward's own decisions: each key tile of the
        // workgroup that the step visits (for a second tile, when it exists and
        // the block holds a row that sees it)
#pragma unroll
        for (int tt = 0; tt < KT_PER; ++tt) {
            const int ktt = kt + tt, jt = j0 + BK * tt;
            if (tt > 0 && (jt >= Lk || qb < (jt - off > 0 ? jt - off : 0) / BQ)) continue;
            if (tid == 0) {
                if (p.kept_tiles) atomicAdd(p.kept_tiles + bh * p.nQB + qb, 1);
                if (p.bits) atomicOr(p.bits + (bh * p.nQB + qb) * p.nwords + (ktt >> 5), 1u << (ktt & 31));
            }
            if (p.kept_slots && tid < BQ) {
                const int i = qb * BQ + tid;
                const int last = off + i - jt;
                if (i < L && last >= 0)
                    atomicAdd(p.kept_slots + sv.lse0 + h * sv.lse_hs + i, (last < BK - 1 ? last : BK - 1) + 1);
            }
        }
        __syncthreads();                         // every wave is done with buffer `buf`
        const int n2 = (nxt >= 0) ? next_step() : -1;
        if (n2 >= 0) fetch(n2, buf);
        wait_prev(n2 >= 0);                      // the next step's blocks have landed
        __syncthreads();
        cur = nxt;
        nxt = n2;
    }

    // ---- epilogue: combine the two query halves (WIDE: each wave holds all
    // of its keys' sums), write dK (scaled) and dV
    __syncthreads();
    float* red = reinterpret_cast<float*>(sU);
    if (!WIDE && qh0 == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                red[(((kw * 2 + 0) * DT + dt) * 16 + r) * 64 + lane] = dv[dt][r];
                red[(((kw * 2 + 1) * DT + dt) * 16 + r) * 64 + lane] = dk[dt][r];
            }
    }
    __syncthreads();
    if (WIDE || qh0 == 0) {
        if (!WIDE)
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
                if (j < Lk) {
                    const int d = 32 * dt + l32;
                    sv.dv[(int64_t)j * p.dv_sl + kh * p.dv_sh + d] = (uint16_t)float_to_bf16_bits(dv[dt][r]);
                    sv.dk[(int64_t)j * p.dk_sl + kh * p.dk_sh + d] =
                        (uint16_t)float_to_bf16_bits(dk[dt][r] * p.scale);
                }
            }
    }
}

// dQ pass: see the file comment.  dQ_i = scale * sum over kept tiles of
// dS_ij k_j, with dS = P (dP - D), P = exp(S - LSE).
template <int D, int BQ, bool VARLEN>
__global__ __launch_bounds__(BQ / 32 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mala_bwd_dq(const BwdParams p) {
    constexpr int NW = BQ / 32;
    constexpr int KSTEPS = D / 16;
    constexpr int DT = D / 32;
    constexpr int QCH = D / 8;
    constexpr int INST = BK * QCH / (NW * 64);   // copies per lane per tile (each of K, V)
    static_assert(INST * NW * 64 == BK * QCH, "shape");
    __shared__ __attribute__((aligned(16))) uint16_t sK[2][BK * D];   // chunk c of row r at c ^ kswz(r)
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][BK * D];   // chunk c of row r at c ^ (r % QCH)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int u = xcd_unit(blockIdx.x, p.chunk_dq);
    if (u >= p.nunits_dq) return;
    const int nbh = p.B * p.Hq;
    const int qb = p.nQB - 1 - u / nbh;          // longest blocks first
    const int64_t bh = u % nbh;
    const int b = (int)(bh / p.Hq);
    const int h = (int)(bh % p.Hq);
    const int kh = h / p.G;
    const SeqView sv = seq_view<BQ, VARLEN>(p, b);
    const int L = sv.Lq, Lk = sv.Lk, off = sv.off;
    if (qb * BQ >= L) return;                     // past the sequence's queries
    const int i = qb * BQ + 32 * w + l32;         // this lane's query row
    const bool valid = i < L;
    const int rend = (qb * BQ + BQ < L) ? qb * BQ + BQ : L;
    const int kt_first = (off + rend - 1) / BK;
    const float c2 = p.scale_log2;

    // ---- Q and dO fragments (B operands: column = query, 8 consecutive d)
    bf16x8 qf[KSTEPS], gf[KSTEPS];
    {
        const uint16_t* qr = sv.q + (int64_t)(valid ? i : 0) * p.q_sl + h * p.q_sh;
        const uint16_t* gr = sv.dout + (int64_t)(valid ? i : 0) * p.do_sl + h * p.do_sh;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            const u32x4 x = valid ? *(const u32x4*)(qr + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            const u32x4 y = valid ? *(const u32x4*)(gr + 16 * st + 8 * hi) : u32x4{0, 0, 0, 0};
            qf[st] = __builtin_bit_cast(bf16x8, x);
            gf[st] = __builtin_bit_cast(bf16x8, y);
        }
    }
    const float lse2 = valid ? p.rowc[sv.row0 + h * sv.row_hs + i] : 0.f;
    const float dval = valid ? p.rowd[sv.row0 + h * sv.row_hs + i] : 0.f;

    // ---- tile copies: buffer resources from the tile to key L-1 (rows past L read zero)
    uint32_t koff[INST], voff[INST];
#pragma unroll
    for (int n = 0; n < INST; ++n) {
        const int sl = (n * NW + w) * 64 + lane;
        const int r = sl / QCH, pc = sl % QCH;
        koff[n] = (uint32_t)((r * p.k_sl + 8 * (pc ^ kswz<QCH>(r))) * 2);
        voff[n] = (uint32_t)((r * p.v_sl + 8 * (pc ^ (r % QCH))) * 2);
    }
    const uint16_t* kbase = sv.k + kh * p.k_sh;
    const uint16_t* vbase = sv.v + kh * p.v_sh;
    auto fetch = [&](int kt, int buf) {
        const int j0 = kt * BK;
        const __amdgpu_buffer_rsrc_t kr =
            make_rsrc(kbase + (int64_t)j0 * p.k_sl, (uint32_t)(((int64_t)(Lk - 1 - j0) * p.k_sl + D) * 2));
        const __amdgpu_buffer_rsrc_t vr =
            make_rsrc(vbase + (int64_t)j0 * p.v_sl, (uint32_t)(((int64_t)(Lk - 1 - j0) * p.v_sl + D) * 2));
#pragma unroll
        for (int n = 0; n < INST; ++n) {
            buffer16_to_lds(kr, koff[n], reinterpret_cast<unsigned char*>(sK[buf]) + (n * NW + w) * 64 * 16);
            buffer16_to_lds(vr, voff[n], reinterpret_cast<unsigned char*>(sV[buf]) + (n * NW + w) * 64 * 16);
        }
    };

    // ---- kept key tiles of this block, newest first: all legal tiles at tau = 0,
    // else the set bits of the block's word row
    const bool dense = p.log2_tau == kNegInf;
    const uint32_t* qrow = p.qbits + (bh * p.nQB + qb) * p.nwords;
    // Sparse cursor, newest tile first.  The row is read 64 words at a time:
    // lane l holds word wtop - l of the current window, `nz` marks the window's
    // non-zero words not yet taken, and cword holds the bits left of word cwi.
    // A stretch of empty words costs one round trip per 64 words.
    int wtop = kt_first >> 5;
    int cwi = 0;
    uint32_t wmy = 0u, cword = 0u;
    uint64_t nz = 0ull;
    if (!dense) {
        const int wi = wtop - lane;
        wmy = qrow[wi >= 0 ? wi : 0];
        wmy = (wi >= 0) ? wmy : 0u;
        if (lane == 0 && kt_first % 32 != 31) wmy &= (2u << (kt_first % 32)) - 1u;   // tiles past kt_first
        nz = __ballot(wmy != 0u);
    }
    int dnext = kt_first;
    auto next_tile = [&]() -> int {
        if (dense) return dnext >= 0 ? dnext-- : -1;
        while (cword == 0u) {
            if (nz == 0ull) {
                wtop -= 64;
                if (wtop < 0) return -1;
                const int wi = wtop - lane;
                wmy = qrow[wi >= 0 ? wi : 0];
                wmy = (wi >= 0) ? wmy : 0u;
                nz = __ballot(wmy != 0u);
                continue;
            }
            const int l = __builtin_ctzll(nz);
            nz &= nz - 1ull;
            cwi = wtop - l;
            cword = (uint32_t)__builtin_amdgcn_readlane((int)wmy, l);
        }
        const int bpos = 31 - __builtin_clz(cword);
        cword &= ~(1u << bpos);
        return cwi * 32 + bpos;
    };

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
    const int j16 = lane & 15;
    const int dsel = 16 * ((lane >> 4) & 1) + 4 * (j16 & 3);

    int tcur = next_tile();
    int tnext = -1;
    if (tcur >= 0) {
        fetch(tcur, 0);
        tnext = next_tile();
        if (tnext >= 0) fetch(tnext, 1);
        if (tnext >= 0) wait_vmcnt<2 * INST>(); else wait_vmcnt<0>();
        __syncthreads();
    }
    for (int s = 0; tcur >= 0; ++s) {
        const int buf = s & 1;
        const uint16_t* kb = sK[buf];
        const uint16_t* vb = sV[buf];
        const int jo = tcur * BK - off;          // key j0 relative to the row offset: j <= off + i
        // every row of the block sees every key of the tile: no mask
        const bool full = (jo + BK - 1 <= qb * BQ) && (qb * BQ + BQ <= L);
        // Each half of the tile (32 keys) goes through scores, dS and its part
        // of the dQ contraction in turn; the scheduling groups keep the LDS
        // operand reads several MFMAs ahead of their use.
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            // S^T = K Q^T and dP^T = V dO^T (one key per register row, this lane's query)
            f32x16 sc = f32x16{}, dp = f32x16{};
            const int row = 32 * sub + l32;
#pragma unroll
            for (int st = 0; st < KSTEPS; ++st) {
                const bf16x8 a = *(const bf16x8*)(&kb[row * D + 8 * ((2 * st + hi) ^ kswz<QCH>(row))]);
                const bf16x8 vv = *(const bf16x8*)(&vb[row * D + 8 * ((2 * st + hi) ^ (row % QCH))]);
                sc = mfma32x32x16(a, qf[st], sc);
                dp = mfma32x32x16(vv, gf[st], dp);
            }
            {
                constexpr int NM = 2 * KSTEPS, PRE = NM < 6 ? NM : 6;
                __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
                for (int n = 0; n < NM - PRE; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
            }
            // dS^T as the B operand of dQ^T
            bf16x8 dsf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = fast_exp2(__builtin_fmaf(sc[r], c2, -lse2));
                dsf[r >> 3][r & 7] = to_bf16(pr * (dp[r] - dval));
            }
            __builtin_amdgcn_sched_barrier(0);
            if (!full) {
                // a diagonal or ragged tile: dS of the pairs that the causal
                // order or the sequence end rules out becomes 0
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    u32x4 dw = __builtin_bit_cast(u32x4, dsf[hf]);
#pragma unroll
                    for (int k2 = 0; k2 < 4; ++k2) {
                        uint32_t m = 0;
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int r = 8 * hf + 2 * k2 + hh;
                            const int j = jo + 32 * sub + 8 * (r >> 2) + 4 * hi + (r & 3);
                            if (valid && j <= i) m |= 0xFFFFu << (16 * hh);
                        }
                        dw[k2] &= m;
                    }
                    dsf[hf] = __builtin_bit_cast(bf16x8, dw);
                }
            }
            // dQ^T += K^T dS^T over this half's keys, K^T fragments (8 keys of
            // one d per lane) by transposing reads
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    const int ks = 2 * sub + kq;
                    u32x2 half2x[2];
#pragma unroll
                    for (int rd = 0; rd < 2; ++rd) {
                        const int krow = 16 * ks + 8 * rd + 4 * hi + (j16 >> 2);
                        const int col = 32 * dt + dsel;
                        const int phys = ((col >> 3) ^ kswz<QCH>(krow)) * 8 + (col & 7);
                        half2x[rd] = lds_read_tr16(kb + krow * D + phys);
                    }
                    // whole-dword assembly of the operand
                    const u32x4 w4 = {half2x[0][0], half2x[0][1], half2x[1][0], half2x[1][1]};
                    acc[dt] = mfma32x32x16(__builtin_bit_cast(bf16x8, w4), dsf[kq], acc[dt]);
                }
            {
                constexpr int NM = 2 * DT, PRE = 4;
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * PRE, 0);
#pragma unroll
                for (int n = 0; n < NM - PRE; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();                         // every wave is done with buffer `buf`
        const int tn2 = (tnext >= 0) ? next_tile() : -1;
        if (tn2 >= 0) fetch(tn2, buf);
        // the tile in the other buffer (copied one step ago) must have landed
        if (tn2 >= 0) wait_vmcnt<2 * INST>(); else wait_vmcnt<0>();
        __syncthreads();
        tcur = tnext;
        tnext = tn2;
    }

    // ---- dQ = scale * acc, C[i = d][j = query]: registers = 4 consecutive d
    if (valid) {
        uint16_t* orow = sv.dq + (int64_t)i * p.dq_sl + h * p.dq_sh;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * dt + 8 * g + 4 * hi;
                u32x2 pk;
                pk[0] = float_to_bf16_bits(acc[dt][4 * g + 0] * p.scale) |
                        (float_to_bf16_bits(acc[dt][4 * g + 1] * p.scale) << 16);
                pk[1] = float_to_bf16_bits(acc[dt][4 * g + 2] * p.scale) |
                        (float_to_bf16_bits(acc[dt][4 * g + 3] * p.scale) << 16);
                *(u32x2*)(orow + d0) = pk;
            }
        }
    }
}

// The packed variable-length layout is a template parameter, so the kernels of
// the fixed-length layout see a zero row offset at compile time.
template <int D, int BQ, bool VARLEN>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
    hipLaunchKernelGGL((mala_bwd_pre<D, BQ, VARLEN>), dim3(p.Lpad / PRE_ROWS, p.Hq, p.B), dim3(256), 0, s, p);
    if (p.log2_tau != -INFINITY) {
        const int per_s = 8 * p.chunk_scan;
        const int grid_s = (p.nunits_scan + per_s - 1) / per_s * per_s;
        hipLaunchKernelGGL((mala_bwd_scan<D, BQ, VARLEN>), dim3(grid_s), dim3(256), 0, s, p);
    }
    // dK / dV: at tau = 0 two key tiles per workgroup (every step is kept, so
    // both tiles use each streamed block) when that still leaves a workgroup
    // for every CU; otherwise one, over its kept steps.  The grid covers the
    // units padded to whole chunks (the tau = 0 order; see the kernel).
    const int per = 8 * p.chunk;
    const int nbk = p.B * p.Hkv;
    const bool wide = p.log2_tau == -INFINITY && nbk * ((p.nKT + 1) / 2) >= p.ncu;
    const int nKTu = wide ? (p.nKT + 1) / 2 : p.nKT;
    const int nu = (nKTu + p.chunk - 1) / p.chunk * p.chunk * nbk;
    const int grid = (nu + per - 1) / per * per;
    if (wide)
        hipLaunchKernelGGL((mala_bwd_kernel<D, BQ, VARLEN, true>), dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((mala_bwd_kernel<D, BQ, VARLEN, false>), dim3(grid), dim3(256), 0, s, p);
    const int per_q = 8 * p.chunk_dq;
    const int grid_q = (p.nunits_dq + per_q - 1) / per_q * per_q;
    hipLaunchKernelGGL((mala_bwd_dq<D, BQ, VARLEN>), dim3(grid_q), dim3(BQ / 32 * 64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, int Bq, int Bk, hipStream_t s) {
    const bool vl = p.cu_q != nullptr;
    if (d == 128 && Bq == 128 && Bk == 64)
        return vl ? launch_bwd_t<128, 128, true>(p, s) : launch_bwd_t<128, 128, false>(p, s);
    if (d == 64 && Bq == 64 && Bk == 64)
        return vl ? launch_bwd_t<64, 64, true>(p, s) : launch_bwd_t<64, 64, false>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace mala
