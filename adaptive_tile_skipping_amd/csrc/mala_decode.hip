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
//   mala_dec_score   one wave per (sequence, KV head, tile): S^T = K q^T with
//                    32x32x16 bf16 MFMAs (the G rows padded to 32 columns),
//                    per-row tile max and shifted sum, base-2 scores spilled
//                    to the workspace.  Reads every K byte once: this is the
//                    HBM-bound score discovery.
//   mala_dec_decide  one wave per (sequence, KV head): the sequential scan.
//                    The row state only grows, so a tile that votes skip under
//                    the current state is skipped; the scan evaluates 64 tiles
//                    per ballot and jumps to the first keeping lane, costing one
//                    step per kept tile plus one per 64 tiles.
//   mala_dec_pv      kept tiles only, split over workgroups: P = 2^(s - lse)
//                    from the spill, V tile loads, fp32 accumulation.
//   mala_dec_combine sums the split partials, writes o (bf16) and LSE.
// tau = 0 keeps every tile, so the scan is elided: mala_dec_dense is a fused
// split-K decode (scores, online softmax and P.V per split) and
// mala_dec_dense_combine merges the splits.
#include "mala_device.h"
#include "mala_internal.h"

namespace mala {

namespace {
constexpr int BKD = 64;
constexpr int GMAX = 16;
}  // namespace

// q fragments for S^T = K q^T: B operand column = row g (lanes g < G), d in a
// permuted order: lane half hi, step st covers d = (D/2)*hi + 8*st .. +8, which
// lets each lane read one contiguous run of its key row.
template <int D>
__device__ __forceinline__ void load_q_frags(const DecParams& p, int b, int kh, bf16x8* qf) {
    constexpr int ST = D / 16;
    const int lane = threadIdx.x & 63;
    const int g = lane & 31, hi = lane >> 5;
    const bool ok = g < p.G;
    const uint16_t* qrow = p.q + ((int64_t)b * p.Hq + kh * p.G + (ok ? g : 0)) * D + (D / 2) * hi;
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        const u32x4 x = ok ? *(const u32x4*)(qrow + 8 * st) : u32x4{0, 0, 0, 0};
        qf[st] = __builtin_bit_cast(bf16x8, x);
    }
}

// Scores of one 64-key tile for the wave: s[sub][r] is row g = lane%32, key
// 32*sub + 8(r/4) + 4*hi + r%4, base 2, -inf past N.
template <int D>
__device__ __forceinline__ void tile_scores(const DecParams& p, int b, int kh, int t, const bf16x8* qf,
                                            f32x16* s) {
    constexpr int ST = D / 16;
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const uint16_t* kb = p.k + b * p.k_sb + kh * p.k_sh;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        int j = t * BKD + 32 * sub + l32;
        j = j < p.N ? j : p.N - 1;
        const uint16_t* kr = kb + (int64_t)j * p.k_sl + (D / 2) * hi;
        u32x4 kx[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st) kx[st] = *(const u32x4*)(kr + 8 * st);
        s[sub] = f32x16{};
#pragma unroll
        for (int st = 0; st < ST; ++st) s[sub] = mfma32x32x16(__builtin_bit_cast(bf16x8, kx[st]), qf[st], s[sub]);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = t * BKD + 32 * sub + 8 * (r >> 2) + 4 * hi + (r & 3);
            s[sub][r] = (j < p.N) ? s[sub][r] * p.scale_log2 : kNegInf;
        }
}

template <int D>
__global__ __launch_bounds__(256) void mala_dec_score(const DecParams p) {
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (task >= p.B * p.Hkv * p.nT) return;
    const int grp = task / p.nT;
    const int t = task % p.nT;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    if (p.bits && lane == 0 && (t % 32) == 0) p.bits[(int64_t)grp * p.nwords + t / 32] = 0u;
    bf16x8 qf[D / 16];
    load_q_frags<D>(p, b, kh, qf);
    f32x16 s[2];
    tile_scores<D>(p, b, kh, t, qf, s);
    float M = kNegInf;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) M = fmaxf(M, s[sub][r]);
    M = wave_max_pair(M);
    float sum = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(s[sub][r] - M);
    sum = wave_sum_pair(sum);
    const int g = l32;
    if (g < p.G) {
        float* sp = p.spill + ((int64_t)grp * p.G + g) * p.N + (int64_t)t * BKD;
        const bool full = (t + 1) * BKD <= p.N;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int j0 = 32 * sub + 8 * q4 + 4 * hi;
                if (full) {
                    *(f32x4*)(sp + j0) = f32x4{s[sub][4 * q4], s[sub][4 * q4 + 1], s[sub][4 * q4 + 2], s[sub][4 * q4 + 3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (t * BKD + j0 + e < p.N) sp[j0 + e] = s[sub][4 * q4 + e];
                }
            }
        if (hi == 0) {
            p.tmax[((int64_t)grp * p.nT + t) * p.G + g] = M;
            p.tsum[((int64_t)grp * p.nT + t) * p.G + g] = sum;
        }
    }
}

__global__ __launch_bounds__(64) void mala_dec_decide(const DecParams p) {
    const int grp = blockIdx.x;
    const int lane = threadIdx.x;
    const int G = p.G;
    const float theta = p.log2_tau - p.log2_N;
    float m[GMAX], l[GMAX], thr[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) { m[g] = kNegInf; l[g] = 0.f; thr[g] = kNegInf; }
    int kept = 0;
    int32_t* klist = p.klist + (int64_t)grp * p.nT;
    const int nchunk = (p.nT + 63) / 64;
    for (int c = 0; c < nchunk; ++c) {
        const int t = p.nT - 1 - (c * 64 + lane);        // newest first
        const bool valid = t >= 0;
        float Mg[GMAX], Sg[GMAX];
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            Mg[g] = kNegInf;
            Sg[g] = 0.f;
            if (g < G && valid) {
                Mg[g] = p.tmax[((int64_t)grp * p.nT + t) * G + g];
                Sg[g] = p.tsum[((int64_t)grp * p.nT + t) * G + g];
            }
        }
        int pos = 0;
        while (pos < 64) {
            bool vote = false;
            if (valid && lane >= pos) {
#pragma unroll
                for (int g = 0; g < GMAX; ++g)
                    if (g < G) vote |= (l[g] == 0.f) || (Mg[g] >= thr[g]);
            }
            const uint64_t mask = __ballot(vote);
            if (mask == 0ull) break;
            const int f = __builtin_ctzll(mask);
#pragma unroll
            for (int g = 0; g < GMAX; ++g) {
                if (g < G) {
                    const float Mf = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Mg[g]), f));
                    const float Sf = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Sg[g]), f));
                    const float mn = fmaxf(m[g], Mf);
                    const float a = (m[g] == kNegInf) ? 0.f : fast_exp2(m[g] - mn);
                    l[g] = l[g] * a + Sf * fast_exp2(Mf - mn);
                    m[g] = mn;
                    thr[g] = m[g] + fast_log2(l[g]) + theta;
                }
            }
            if (lane == 0) {
                const int tk = p.nT - 1 - (c * 64 + f);
                klist[kept] = tk;
                if (p.bits) atomicOr(p.bits + (int64_t)grp * p.nwords + tk / 32, 1u << (tk % 32));
            }
            ++kept;
            pos = f + 1;
        }
    }
    if (lane == 0) {
        p.kcount[grp] = kept;
        if (p.kept_tiles) p.kept_tiles[grp] = kept;
    }
    if (lane < G) {
        float mm = kNegInf, ll = 0.f;
#pragma unroll
        for (int g = 0; g < GMAX; ++g)
            if (g == lane) { mm = m[g]; ll = l[g]; }
        const float lz2 = mm + fast_log2(ll);
        p.lse2[(int64_t)grp * G + lane] = lz2;
        const int b = grp / p.Hkv, kh = grp % p.Hkv;
        p.lse[(int64_t)b * p.Hq + kh * G + lane] = lz2 * kLn2;
    }
}

// Thread layout of the P.V phase: dc = tid % (D/8) owns d = 8 dc .. 8 dc + 7,
// kg = tid / (D/8) owns keys kg*KPT .. of each tile.
template <int D>
__global__ __launch_bounds__(256) void mala_dec_pv(const DecParams p) {
    constexpr int DC = D / 8;
    constexpr int NKG = 256 / DC;          // key groups
    constexpr int KPT = BKD / NKG;         // keys per thread per tile
    __shared__ float sP[GMAX][BKD];
    __shared__ float sRed[NKG][D];
    const int tid = threadIdx.x;
    const int s = blockIdx.x, grp = blockIdx.y;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    const int G = p.G;
    const int cnt = p.kcount[grp];
    const int per = (cnt + p.nsplit - 1) / p.nsplit;
    const int i0 = s * per;
    const int i1 = (i0 + per < cnt) ? i0 + per : cnt;
    const int dc = tid % DC, kg = tid / DC;
    float acc[GMAX][8];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    const uint16_t* vb = p.v + b * p.v_sb + kh * p.v_sh + 8 * dc;
    for (int idx = i0; idx < i1; ++idx) {
        const int t = p.klist[(int64_t)grp * p.nT + idx];
        for (int e = tid; e < G * BKD; e += 256) {
            const int g = e / BKD, j = e % BKD;
            const int key = t * BKD + j;
            float pr = 0.f;
            if (key < p.N)
                pr = fast_exp2(p.spill[((int64_t)grp * G + g) * p.N + key] - p.lse2[(int64_t)grp * G + g]);
            sP[g][j] = pr;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int j = kg * KPT + r;
            int key = t * BKD + j;
            key = key < p.N ? key : p.N - 1;      // P is 0 past N
            const u32x4 x = *(const u32x4*)(vb + (int64_t)key * p.v_sl);
            float vv[8];
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2) {
                vv[2 * m2] = __uint_as_float(x[m2] << 16);
                vv[2 * m2 + 1] = __uint_as_float(x[m2] & 0xFFFF0000u);
            }
#pragma unroll
            for (int g = 0; g < GMAX; ++g) {
                if (g < G) {
                    const float pr = sP[g][j];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[g][e] += pr * vv[e];
                }
            }
        }
        __syncthreads();
    }
    // reduce over key groups, one row at a time
    float* po = p.part_o + (((int64_t)grp * p.nsplit + s) * G) * D;
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int gg = 0; gg < GMAX; ++gg)
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
}

template <int D>
__global__ __launch_bounds__(256) void mala_dec_combine(const DecParams p) {
    const int grp = blockIdx.x;
    const int G = p.G;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    for (int e = threadIdx.x; e < G * D; e += 256) {
        const int g = e / D, d = e % D;
        float sum = 0.f;
        for (int s = 0; s < p.nsplit; ++s) sum += p.part_o[(((int64_t)grp * p.nsplit + s) * G + g) * D + d];
        p.o[((int64_t)b * p.Hq + kh * G + g) * D + d] = (uint16_t)float_to_bf16_bits(sum);
    }
}

// tau = 0: fused split-K decode.  Each workgroup owns tiles_per_split tiles of
// one (sequence, KV head); its 4 waves score 4 tiles at a time, then the whole
// workgroup runs the online-softmax update and P.V for those 256 keys.
template <int D>
__global__ __launch_bounds__(256) void mala_dec_dense(const DecParams p) {
    constexpr int DC = D / 8;
    constexpr int NKG = 256 / DC;
    constexpr int KPT = 4 * BKD / NKG;     // keys per thread per group of 4 tiles
    __shared__ float sS[GMAX][4 * BKD];
    __shared__ float sAlpha[GMAX];
    __shared__ float sState[GMAX][2];      // running max, sum
    __shared__ float sRed[NKG][D];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int s = blockIdx.x, grp = blockIdx.y;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    const int G = p.G;
    const int t0 = s * p.tiles_per_split;
    const int t1 = (t0 + p.tiles_per_split < p.nT) ? t0 + p.tiles_per_split : p.nT;
    bf16x8 qf[D / 16];
    load_q_frags<D>(p, b, kh, qf);
    if (tid < GMAX) { sState[tid][0] = kNegInf; sState[tid][1] = 0.f; }
    const int dc = tid % DC, kg = tid / DC;
    float acc[GMAX][8];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    const uint16_t* vb = p.v + b * p.v_sb + kh * p.v_sh + 8 * dc;
    __syncthreads();
    for (int tb = t0; tb < t1; tb += 4) {
        // ---- scores of tiles tb .. tb+3 (wave w: tile tb + w)
        {
            const int t = tb + w;
            f32x16 sc[2];
            if (t < t1) {
                tile_scores<D>(p, b, kh, t, qf, sc);
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
        // ---- online softmax over the 256 new scores: 16 threads per row
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
        // ---- P.V over the 4 tiles' keys
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g < G) {
                const float a = sAlpha[g];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] *= a;
            }
        }
        for (int r = 0; r < KPT; ++r) {
            const int jj = kg * KPT + r;                 // 0 .. 255 within the 4 tiles
            int key = tb * BKD + jj;
            if (key >= t1 * BKD || key >= p.N) continue;
            const u32x4 x = *(const u32x4*)(vb + (int64_t)key * p.v_sl);
            float vv[8];
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2) {
                vv[2 * m2] = __uint_as_float(x[m2] << 16);
                vv[2 * m2 + 1] = __uint_as_float(x[m2] & 0xFFFF0000u);
            }
#pragma unroll
            for (int g = 0; g < GMAX; ++g) {
                if (g < G) {
                    const float pr = sS[g][jj];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[g][e] += pr * vv[e];
                }
            }
        }
        __syncthreads();
    }
    float* po = p.part_o + (((int64_t)grp * p.nsplit + s) * G) * D;
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int gg = 0; gg < GMAX; ++gg)
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

template <int D>
__global__ __launch_bounds__(256) void mala_dec_dense_combine(const DecParams p) {
    const int grp = blockIdx.x;
    const int G = p.G;
    const int b = grp / p.Hkv, kh = grp % p.Hkv;
    for (int e = threadIdx.x; e < G * D; e += 256) {
        const int g = e / D, d = e % D;
        float M = kNegInf;
        for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, p.part_ml[(((int64_t)grp * p.nsplit + s) * G + g) * 2]);
        float lsum = 0.f, osum = 0.f;
        for (int s = 0; s < p.nsplit; ++s) {
            const int64_t ix = ((int64_t)grp * p.nsplit + s) * G + g;
            const float ms = p.part_ml[ix * 2];
            if (ms == kNegInf) continue;
            const float a = fast_exp2(ms - M);
            lsum += p.part_ml[ix * 2 + 1] * a;
            osum += p.part_o[ix * D + d] * a;
        }
        p.o[((int64_t)b * p.Hq + kh * G + g) * D + d] = (uint16_t)float_to_bf16_bits(osum / lsum);
        if (d == 0) p.lse[(int64_t)b * p.Hq + kh * G + g] = (M + fast_log2(lsum)) * kLn2;
    }
    if (threadIdx.x == 0 && p.kept_tiles) p.kept_tiles[grp] = p.nT;
    if (p.bits)
        for (int wd = threadIdx.x; wd < p.nwords; wd += 256) {
            const int rem = p.nT - 32 * wd;
            p.bits[(int64_t)grp * p.nwords + wd] = rem >= 32 ? 0xFFFFFFFFu : ((1u << rem) - 1u);
        }
}

template <int D>
static hipError_t launch_decode_t(const DecParams& p, bool dense, hipStream_t s) {
    const int ngrp = p.B * p.Hkv;
    if (dense) {
        hipLaunchKernelGGL((mala_dec_dense<D>), dim3(p.nsplit, ngrp), dim3(256), 0, s, p);
        hipLaunchKernelGGL((mala_dec_dense_combine<D>), dim3(ngrp), dim3(256), 0, s, p);
    } else {
        const int tasks = ngrp * p.nT;
        hipLaunchKernelGGL((mala_dec_score<D>), dim3((tasks + 3) / 4), dim3(256), 0, s, p);
        hipLaunchKernelGGL(mala_dec_decide, dim3(ngrp), dim3(64), 0, s, p);
        hipLaunchKernelGGL((mala_dec_pv<D>), dim3(p.nsplit, ngrp), dim3(256), 0, s, p);
        hipLaunchKernelGGL((mala_dec_combine<D>), dim3(ngrp), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecParams& p, int d, int Bkd, bool dense, hipStream_t s) {
    if (Bkd != BKD || p.G > GMAX) return hipErrorInvalidValue;
    if (d == 128) return launch_decode_t<128>(p, dense, s);
    if (d == 64) return launch_decode_t<64>(p, dense, s);
    return hipErrorInvalidValue;
}

}  // namespace mala
