/*
 * libmala -- MALA (MassAlloc Attention) fused causal attention for AMD MI355X
 * (gfx950).  C ABI: plain pointers, sizes and element strides; no C++ or
 * framework types cross it, no exception leaves it.
 *
 * The operation ("MassAlloc Attention: Let Attention Allocate Its Own
 * Compute", arXiv 2609.32712; summary page agihunt.info, and review page
 * jaehun.me, sections "One tolerance governs everything", "Forward: online
 * sparse softmax", "Backward: offline sparse probabilities"):
 *   causal softmax attention in which every legal query-key tile is scored,
 *   but the post-score work of a tile (softmax update, V load, P.V) is skipped
 *   when, for every row of the query block, exp(tile row max) divided by the
 *   softmax mass retained so far is below tau / L_i, L_i = i + 1 being the
 *   number of keys row i can see.  Tiles are visited from the diagonal toward
 *   key 0, so the first legal tile of each row is always kept (its retained
 *   mass is still empty).  The backward pass re-applies the test with the
 *   final log-normaliser (LSE) saved by the forward, so its kept set is a
 *   subset of the forward's; no mask is stored.  tau = 0 skips nothing and is
 *   plain causal softmax attention.
 *
 * Conventions shared by every entry point:
 *   - Tensors are bf16 (IEEE bfloat16, round-to-nearest-even), described by
 *     mala_t4: element pointer and element strides for dims [B, L, H, d]; the d
 *     dimension is contiguous.  Pointers and the byte size of every stride must
 *     be 16-byte aligned (strides multiples of 8 elements).
 *   - Scale is 1/sqrt(d); LSE is the natural log of the retained normaliser of
 *     the scaled scores.
 *   - GQA: Hq must be a multiple of Hkv; q head h reads KV head h / (Hq/Hkv).
 *   - The caller owns every buffer, including workspaces; the library
 *     allocates no device memory.  Its only global state is written once per
 *     device and then only read: a cache of the device's compute-unit count,
 *     and the device address of mala_decode_noalloc's fixed scratch array
 *     (that array, one per GPU, is the one buffer the library owns).
 *     Concurrent first calls store the same values.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting.  Arguments are validated on the host
 *     before anything is enqueued: an invalid call enqueues nothing.
 *   - tau must be finite and >= 0.
 *   - Arithmetic: scores, softmax state and accumulators in fp32; the other
 *     contractions take bf16 operands, except the forward's P.V, which runs in
 *     fp16: P in [0, 1] rounded to nearest, and V converted from bf16 to fp16
 *     rounding toward zero.  That conversion is exact for v = 0 and for
 *     2^-17 <= |v| <= 65504 (every bf16 value there is an fp16 value); a
 *     smaller |v| is truncated toward zero to a multiple of 2^-24 (to 0 below
 *     2^-24), and a larger one becomes +-65504.  Keep V inside that range for
 *     mala_fwd (rescale it otherwise); mala_bwd and the decode read bf16 V as
 *     is.  The decode's P.V takes P as fp16 values split exactly into two bf16
 *     parts, against bf16 V.
 *   - Supported shapes: (d, Bq, Bk) = (128, 128, 64) or (64, 64, 64) for
 *     mala_fwd / mala_bwd; decode takes d = 128 or 64 with Bk_dec = 64.
 *     Byte ranges addressed through 32-bit buffer resources must stay within
 *     INT32_MAX: mala_fwd needs ((L-1) * k's L stride + d) * 2 and
 *     (L + Bq) * d * 2; mala_bwd needs (Bq * q's L stride + d) * 2 and
 *     (Bk * k's L stride + d) * 2.
 *     Anything else returns MALA_ERR_UNSUPPORTED.
 */
#ifndef MALA_H_
#define MALA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MALA_OK = 0,
    MALA_ERR_INVALID_ARG = 1,   /* null required pointer, bad shape/stride/alignment, bad tau */
    MALA_ERR_UNSUPPORTED = 2,   /* (d, Bq, Bk) combination not built, or a stride beyond a kernel's range */
    MALA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the *_workspace_size query */
    MALA_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} mala_status;

/* A bf16 tensor [B, L, H, d]; element strides; d stride is 1. */
typedef struct {
    void* ptr;
    int64_t sb, sl, sh;
} mala_t4;

/* A packed bf16 tensor [total, H, d] of variable-length sequences (rows of
 * all sequences back to back); element strides; d stride is 1. */
typedef struct {
    void* ptr;
    int64_t sl, sh;
} mala_t3;

/* Optional per-call tile statistics (every pointer may be NULL).
 *   kept_tiles    [B, Hq, nQB] int32: retained key tiles per query block.
 *   kept_slots    [B, Hq, L]   int32: legal (causal) keys inside retained
 *                 tiles, per row -- the post-score key slots of the row.
 *   omitted_mass  [B, Hq, L]   fp32: probability mass of the skipped legal
 *                 keys, Z_O / (Z_R + Z_O).  Non-NULL switches the kernel to
 *                 a statistics mode that also exponentiates skipped tiles
 *                 (slower; keep NULL in timed runs).  Forward only.
 *   decision_bits [B, Hq, nQB, ceil(nKT/32)] uint32: bit (kt % 32) of word
 *                 kt / 32 is 1 iff key tile kt was retained for the block;
 *                 bits of tiles the block never visits are 0.
 * nQB = ceil(L / Bq), nKT = ceil(L / Bk).  Every element is overwritten. */
typedef struct {
    int32_t* kept_tiles;
    int32_t* kept_slots;
    float* omitted_mass;
    uint32_t* decision_bits;
} mala_tile_stats;

/* Bytes of device workspace mala_fwd needs (an fp16 copy of V and the forward
 * kernel's work queues).  Calls that overlap in time need separate workspaces. */
size_t mala_fwd_workspace_size(int B, int L, int Hq, int Hkv, int d, int Bq, int Bk);

/* Forward (training forward or prefill), causal, Lq = Lk = L.
 *   q [B, L, Hq, d], k, v [B, L, Hkv, d] bf16 in device memory.
 *   o [B, L, Hq, d] bf16 output; lse [B, Hq, L] fp32 output (contiguous).
 *   stats: NULL or per-call statistics (see mala_tile_stats).
 *   ws: device workspace of at least mala_fwd_workspace_size(...) bytes,
 *   256-byte aligned; overwritten by the call.
 * Decision rule: review page "Forward: online sparse softmax"; summary page,
 * forward paragraph. */
mala_status mala_fwd(mala_t4 q, mala_t4 k, mala_t4 v, int B, int L, int Hq, int Hkv, int d,
                     float tau, int Bq, int Bk, mala_t4 o, float* lse,
                     const mala_tile_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace mala_fwd_varlen needs (an fp16 copy of V with
 * room for Bk more keys after each sequence, and the forward kernel's work
 * queues). */
size_t mala_fwd_varlen_workspace_size(int B, int total_k, int Hkv, int d, int Bq, int Bk);

/* Forward over a packed batch of B variable-length sequences, each a chunk of
 * Lq queries over Lk >= Lq keys: prompt prefill (Lq = Lk), chunked prefill
 * onto an existing cache (Lq < Lk) and mixed batches of both.  The queries
 * are the last Lq positions of the sequence (bottom-right causal alignment):
 * query row i of the chunk sees keys j <= Lk - Lq + i, so L_i = Lk - Lq + i + 1
 * in the decision rule.  Key tiles are aligned to key 0 and query blocks to
 * the chunk's first row, so a chunk that starts at a multiple of Bq gives the
 * rows mala_fwd gives for the whole sequence.  (Summary page: prefill is a
 * mode under the same tau; review page "One tolerance governs everything":
 * the threshold tau / L_i uses the row's visible-key count.)
 *   q [total_q, Hq, d], k, v [total_k, Hkv, d] bf16 (mala_t3), in device memory.
 *   cu_seqlens_q, cu_seqlens_k: int32 [B + 1] in DEVICE memory, cumulative
 *   lengths (cu[0] = 0, cu[B] = total): sequence b owns query rows
 *   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 *   cu_seqlens_k[b+1]-1.  They are read by the kernels, not on the host: a
 *   sequence whose lengths break 0 <= Lq <= Lk, Lq <= max_seqlen_q,
 *   Lk <= max_seqlen_k, or whose rows leave [0, total) is skipped and its
 *   outputs are left unwritten (no out-of-range access is made).
 *   o [total_q, Hq, d] bf16 output; lse [Hq, total_q] fp32 output (contiguous).
 *   stats: NULL or statistics as for mala_fwd, with nQB = ceil(max_seqlen_q /
 *   Bq) and nKT = ceil(max_seqlen_k / Bk) (kept_tiles and decision_bits indexed
 *   [B, Hq, nQB, ...], 0 for blocks past a sequence's queries; kept_slots and
 *   omitted_mass [Hq, total_q]).
 *   ws: device workspace of at least mala_fwd_varlen_workspace_size(...)
 *   bytes, 256-byte aligned; overwritten by the call.
 * INVALID_ARG for bad sizes (max_seqlen_q > max_seqlen_k, a maximum above its
 * total, negative counts) besides the shared conditions; UNSUPPORTED when
 * B > 65535 or when ((max_seqlen_k - 1) * k's L stride + d) * 2 or
 * (max_seqlen_k + Bk) * d * 2 exceeds INT32_MAX.  total_q = 0 returns MALA_OK and enqueues nothing. */
mala_status mala_fwd_varlen(mala_t3 q, mala_t3 k, mala_t3 v, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int B, int total_q, int total_k, int max_seqlen_q,
                            int max_seqlen_k, int Hq, int Hkv, int d, float tau, int Bq, int Bk, mala_t3 o,
                            float* lse, const mala_tile_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace mala_bwd needs (row terms and kept-tile bits). */
size_t mala_bwd_workspace_size(int B, int L, int Hq, int Hkv, int d, int Bq, int Bk);

/* Backward.  Inputs as saved by mala_fwd (q, k, v, o, lse) plus dout.
 *   dq [B, L, Hq, d], dk, dv [B, L, Hkv, d] bf16 outputs (dk/dv summed over
 *   the q heads of each KV head).  ws: device workspace of at least
 *   mala_bwd_workspace_size(...) bytes, 256-byte aligned; it is cleared by the
 *   call itself (on the stream) and may be reused between calls.
 *   bwd_stats: NULL or statistics of the backward's own decisions
 *   (kept_tiles, kept_slots, decision_bits; omitted_mass must be NULL).
 * Decision rule: review page "Backward: offline sparse probabilities";
 * summary page, backward paragraph.  The result is not the exact derivative
 * of the forward for tau > 0 (the pages say so); it is the softmax-attention
 * gradient restricted to the tiles the backward keeps. */
mala_status mala_bwd(mala_t4 q, mala_t4 k, mala_t4 v, mala_t4 o, mala_t4 dout, const float* lse,
                     int B, int L, int Hq, int Hkv, int d, float tau, int Bq, int Bk,
                     mala_t4 dq, mala_t4 dk, mala_t4 dv, void* ws, size_t ws_bytes,
                     const mala_tile_stats* bwd_stats, void* stream);

/* Bytes of device workspace mala_bwd_varlen needs (row terms with Bq rows of
 * padding per sequence, and kept-tile bits). */
size_t mala_bwd_varlen_workspace_size(int B, int total_q, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv,
                                      int d, int Bq, int Bk);

/* Backward of mala_fwd_varlen over the same packed batch: training on packed
 * sequences (Lq = Lk per sequence) and on chunks whose queries sit at the end
 * of their keys.  Same rule as mala_bwd with L_i = Lk - Lq + i + 1 (review
 * page "Backward: offline sparse probabilities"; summary page, backward
 * paragraph).
 *   q, o, dout [total_q, Hq, d]; k, v [total_k, Hkv, d] bf16 (mala_t3); lse
 *   [Hq, total_q] fp32 as written by mala_fwd_varlen; cu_seqlens_q/_k int32
 *   [B + 1] in device memory, read by the kernels (a sequence whose lengths
 *   break the conditions of mala_fwd_varlen is skipped and its gradients are
 *   left unwritten).
 *   dq [total_q, Hq, d], dk, dv [total_k, Hkv, d] bf16 outputs; keys of a
 *   sequence without queries get dk = dv = 0.
 *   ws: at least mala_bwd_varlen_workspace_size(...) bytes, 256-byte aligned,
 *   cleared by the call itself.  bwd_stats: as for mala_bwd, with nQB, nKT from
 *   max_seqlen_q / max_seqlen_k and kept_slots [Hq, total_q].
 * Errors as for mala_fwd_varlen; UNSUPPORTED also when (Bq * q's (or dout's)
 * row stride + d) * 2 or ((max_seqlen_k - 1) * k's (or v's) row stride + d) * 2
 * exceeds INT32_MAX.  total_k = 0 returns MALA_OK and enqueues nothing. */
mala_status mala_bwd_varlen(mala_t3 q, mala_t3 k, mala_t3 v, mala_t3 o, mala_t3 dout, const float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int total_q,
                            int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d, float tau,
                            int Bq, int Bk, mala_t3 dq, mala_t3 dk, mala_t3 dv, void* ws, size_t ws_bytes,
                            const mala_tile_stats* bwd_stats, void* stream);

/* Bytes of device workspace mala_decode needs (tile statistics, score spill,
 * retained-tile lists, partial outputs). */
size_t mala_decode_workspace_size(int B, int N, int Hq, int Hkv, int d, int Bk_dec);

/* Decode: one new query token per sequence against a KV cache of N keys (the
 * cache includes the new token's key and value).
 *   q [B, Hq, d] bf16 contiguous; kcache, vcache [B, N, Hkv, d] bf16 (mala_t4
 *   with L = N).  o [B, Hq, d] bf16 output; lse [B, Hq] fp32 output.
 *   kept_tiles: NULL or [B, Hkv] int32 output, retained cache tiles per
 *   (sequence, KV head).  decision_bits: NULL or [B, Hkv, ceil(nT/32)] uint32
 *   output, nT = ceil(N / Bk_dec): bit (t % 32) of word t / 32 is 1 iff cache
 *   tile t was retained.  ws: device workspace of at least
 *   mala_decode_workspace_size(...) bytes, 256-byte aligned.
 * The decision block is the group of Hq/Hkv q heads sharing a KV head, all
 * with L_i = N; cache tiles of Bk_dec keys are visited newest first (same
 * tau as training: summary page, forward paragraph; review page "One
 * tolerance governs everything"). */
mala_status mala_decode(const void* q, mala_t4 kcache, mala_t4 vcache, int B, int N, int Hq, int Hkv,
                        int d, float tau, int Bk_dec, void* o, float* lse, int32_t* kept_tiles,
                        uint32_t* decision_bits, void* ws, size_t ws_bytes, void* stream);

/* Decode against caches of different lengths per sequence (the cache tensor
 * padded to N rows): sequence b uses its first cache_seqlens[b] rows, which
 * include the new token's key and value, and its decision uses
 * L_i = cache_seqlens[b] (same rule and summary/review passages as
 * mala_decode).  Arguments as for mala_decode, plus:
 *   cache_seqlens: int32 [B] in DEVICE memory, read by the kernels.  A
 *   sequence whose length lies outside [1, N] is skipped: its o and lse are
 *   left unwritten, its kept_tiles entry and decision bits are 0.
 * Cache tiles past a sequence's length are not read; decision_bits of those
 * tiles are 0.  The workspace is mala_decode_workspace_size(B, N, ...).
 * cache_seqlens = NULL returns MALA_ERR_INVALID_ARG. */
mala_status mala_decode_varlen(const void* q, mala_t4 kcache, mala_t4 vcache, const int32_t* cache_seqlens, int B,
                               int N, int Hq, int Hkv, int d, float tau, int Bk_dec, void* o, float* lse,
                               int32_t* kept_tiles, uint32_t* decision_bits, void* ws, size_t ws_bytes,
                               void* stream);

/* Largest workspace mala_decode_noalloc can serve: 64 MiB, enough for
 * mala_decode_workspace_size of 8 sequences x 131072 cached keys x 5 q heads
 * per KV head (about 16 MiB) four times over. */
#define MALA_DECODE_NOALLOC_MAX_BYTES (64u << 20)

/* mala_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results as mala_decode, without ws / ws_bytes: the
 * workspace is a fixed array of MALA_DECODE_NOALLOC_MAX_BYTES in the
 * library's device code, one per GPU, held until the process ends.  Nothing
 * is allocated, by the library or anything it calls.
 *   Calls whose mala_decode_workspace_size(B, N, Hq, Hkv, d, Bk_dec) exceeds
 *   MALA_DECODE_NOALLOC_MAX_BYTES return MALA_ERR_WORKSPACE and enqueue
 *   nothing (after the argument checks of mala_decode, whose errors come
 *   first).  MALA_ERR_HIP if the array's address cannot be found on the
 *   current device (more than 64 devices, or a runtime failure).
 *   Every call on one GPU shares that GPU's array, so calls that may overlap
 *   in time on one GPU (other streams, other threads) race and give wrong
 *   results: serialise them, or use mala_decode with separate workspaces.
 *   Each call writes every part of the array it reads before reading it;
 *   nothing from an earlier call carries over. */
mala_status mala_decode_noalloc(const void* q, mala_t4 kcache, mala_t4 vcache, int B, int N, int Hq, int Hkv,
                                int d, float tau, int Bk_dec, void* o, float* lse, int32_t* kept_tiles,
                                uint32_t* decision_bits, void* stream);

/* Measurement aids, for callers that read the attention kernels' rates
 * against what this part sustains as well as against its published peaks.
 * They compute nothing of the attention method.  Both enqueue one kernel on
 * `stream` and return before it finishes; time them with events on that
 * stream.
 *
 * Words of the sink buffer either probe may write. */
#define MALA_PROBE_SINK_WORDS (256u * 1024u)

/* Back-to-back 32x32x16 bf16 MFMAs on register operands, no memory traffic:
 * a grid of two 4-wave workgroups per compute unit, each wave running
 * `iters` rounds of four independent MFMAs.  mala_probe_mfma_flop(iters) is
 * the launch's FLOP count (2*32*32*16 per MFMA).
 *   sink: DEVICE memory of MALA_PROBE_SINK_WORDS floats (caller-owned);
 *   one value per wave is written to it.
 * MALA_ERR_INVALID_ARG for iters < 1 or a null sink (nothing enqueued);
 * MALA_ERR_HIP if the launch fails. */
mala_status mala_probe_mfma(int iters, float* sink, void* stream);
double mala_probe_mfma_flop(int iters);

/* A plain streaming read of `bytes` bytes at `src` (DEVICE memory, 16-byte
 * aligned, bytes a positive multiple of 16): one 8-wave workgroup per
 * compute unit, grid-stride 16-byte loads, eight in flight per lane.
 *   sink: DEVICE memory of MALA_PROBE_SINK_WORDS uint32 (caller-owned); one
 *   word per thread (the XOR of what it read) is written to it.
 * MALA_ERR_INVALID_ARG for a null pointer, a misaligned src or a bad size
 * (nothing enqueued); MALA_ERR_HIP if the launch fails. */
mala_status mala_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Static string naming a status code. */
const char* mala_status_string(mala_status s);

/* Library version, e.g. "0.1.0 gfx950". */
const char* mala_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MALA_H_ */
