/*
 * fp64 CPU oracle for MALA (MassAlloc Attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is a slow, plain statement
 * of what the method computes, used to check the GPU path.
 *
 * Source: "MassAlloc Attention: Let Attention Allocate Its Own Compute"
 * (arXiv 2609.32712), as described by the pages
 *   [P1] agihunt.info paper summary, paragraphs on the rule (forward, backward,
 *        tau -> 0) and the limitations paragraph (omitted-mass bound);
 *   [P2] jaehun.me review, "New approach: MassAlloc Attention" -> "One tolerance
 *        governs everything", "Forward: online sparse softmax", "Backward:
 *        offline sparse probabilities", "Theoretical upper bound on forward
 *        omitted mass" (Prop. 1), and "How it works: a concrete example".
 *
 * Notation (all 0-indexed): causal self-attention with Lq = Lk = L; row i sees
 * L_i = i + 1 keys ([P1]: the query's visible-key count; [P2] "One tolerance":
 * uniform attention gives each visible key 1/L_q).  Scores s_ij = q_i.k_j/sqrt(d).
 * theta_i = ln tau - ln L_i is the log of the length-normalised threshold
 * tau/L_i; tau = 0 gives theta = -inf, i.e. nothing is ever skipped ([P1]:
 * tau -> 0 recovers full attention).  GQA: q head h reads KV head h / (Hq/Hkv).
 *
 * Readings taken where the pages are silent or garbled (the log-form test on
 * [P2] lost its formula in extraction):
 *   - a row votes to keep tile t iff it has a legal key in t and either its
 *     retained mass is still empty (l_i = 0) or
 *         M_i - m_i - ln l_i >= theta_i,
 *     i.e. exp(tile row max) / (mass retained so far, candidate excluded)
 *     >= tau / L_i.  Equality keeps.  The empty-state case is what makes the
 *     first legal tile always kept ([P1]).
 *   - the block keeps the tile iff any row votes keep ([P1]: skip only if every
 *     valid row is below the threshold).
 *   - a skipped tile leaves m, l and the accumulator untouched ([P2] "Forward").
 *   - backward keeps tile t of a query block iff some row with a legal key has
 *     M_i - LSE_i >= theta_i, with LSE the forward's final log-normaliser
 *     ([P2] "Backward"); no tile is forced and no mask is stored.
 *   - backward uses the standard softmax-attention gradient restricted to the
 *     kept tiles, with D_i = dO_i . o_i from the forward output.
 *   - decode applies the forward rule to the block of the G q heads sharing a
 *     KV head, with L_i = N (the cache includes the new token), tiles of the
 *     cache visited newest first ([P2] "One tolerance": one tau for decoding).
 *   - prefill onto an existing cache (Lq <= Lk; [P1] names prefill as a mode
 *     under the same tau): the Lq queries are the last Lq positions of the
 *     sequence, so query row i (0-indexed in the chunk) sees keys
 *     j <= Lk - Lq + i and L_i = Lk - Lq + i + 1.  Key tiles stay aligned to
 *     key 0 and query blocks start at the chunk's first row, so a chunk that
 *     starts at a multiple of Bq reproduces the rows of the full forward.
 *
 * Layouts: q, o, dout, dq: [B][L][Hq][d]; k, v, dk, dv: [B][L][Hkv][d];
 * lse: [B][Hq][L]; per-tile arrays keep/margin: [B][Hq][nQB][nKT] with
 * nQB = ceil(L/Bq), nKT = ceil(L/Bk).  The variable-length forward packs the
 * sequences instead: q, o [total_q][Hq][d]; k, v [total_k][Hkv][d]; lse,
 * kept_slots, omitted [Hq][total_q]; keep/margin [B][Hq][nQB][nKT] with nQB,
 * nKT taken from the longest query and key lengths.  keep holds 1 (kept) or 0 (skipped) for
 * every visited tile; entries of tiles never visited are not written.
 * margin holds the decision's log-margin
 *     forward:  max over voting rows of (M_i - m_i - ln l_i - theta_i)
 *               (+inf if some row has l_i = 0),
 *     backward: max over rows with a legal key of (M_i - LSE_i - theta_i);
 * the tile is kept iff margin >= 0.
 *
 * Gradient error scales (optional backward outputs dq_cond, dk_cond, same
 * layouts as dq, dk).  They are not part of the method: they size the error an
 * evaluation of the gradient in binary32 arithmetic from bf16 inputs may
 * make.  dS_ij = P_ij (dP_ij - D_i) subtracts two length-d
 * dot products, dP_ij = dO_i . v_j and D_i = dO_i . o_i; summed in binary32
 * from exact products, each errs by at most gamma_d times the same sum of
 * absolute values, gamma_d = d u / (1 - d u), u = 2^-24 (Higham, "Accuracy and
 * Stability of Numerical Algorithms", 2nd ed., section 3.1).  Carried through
 * dq_i = scale sum_j dS_ij k_j and dk_j = scale sum_i dS_ij q_i, that moves
 * the gradients by at most gamma_d times
 *     dq_cond[i][c] = scale sum_j P_ij (|dO_i|.|v_j| + |dO_i|.|o_i|) |k_jc|
 *     dk_cond[j][c] = scale sum_i P_ij (|dO_i|.|v_j| + |dO_i|.|o_i|) |q_ic|
 * to first order (sums over the kept legal pairs; |x|.|y| = sum_c |x_c||y_c|;
 * dk_cond summed over the q heads of the group).  Where dS cancels (a row
 * whose attention sits on one key, so o_i is that key's value) this bound,
 * not the gradient's own norm, is what such an evaluation can resolve.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_EINVAL 1
#define OR_ENOMEM 2

static int tau_valid(double tau) { return isfinite(tau) && tau >= 0.0; }

/* log of the length-normalised threshold tau / L_vis */
static double log_threshold(double tau, double L_vis) {
    if (tau == 0.0) return -INFINITY;
    return log(tau) - log(L_vis);
}

static double dot(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

static double dot_abs(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += fabs(a[c]) * fabs(b[c]);
    return s;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int mala_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Forward ([P2] "Forward: online sparse softmax"; [P1] forward paragraph)    */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *q, *k, *v;
    int B, Hq, Hkv, d, Bq, Bk, nQB, nKT;
    /* per sequence: first packed row of its queries and of its keys, query
     * and key counts, and the base of its [Hq] row-statistics rows */
    const long *qoff, *koff, *lseoff;
    const int *lq, *lk;
    long lse_hstride;   /* distance between heads in lse / kept_slots / omitted */
    double tau, scale;
    double *o, *lse, *margin, *omitted;
    uint8_t* keep;
    int32_t* kept_slots;
    /* NULL, or [B][Hq][nQB][nKT]: 0 / 1 forces the decision a tile's update
     * uses, 255 leaves it to the rule (teacher-forced replay, see
     * mala_oracle_fwd_forced) */
    const uint8_t* forced;
} fwd_ctx;

static int fwd_block(const fwd_ctx* c, int b, int h, int qb) {
    const int d = c->d, Hq = c->Hq, Hkv = c->Hkv, Bk = c->Bk;
    const int Lq = c->lq[b], Lk = c->lk[b];
    const int off = Lk - Lq;          /* keys before the first query of the chunk */
    const int kh = h / (Hq / Hkv);
    const int r0 = qb * c->Bq;
    if (r0 >= Lq) return OR_OK;       /* past this sequence's queries: not visited */
    const int r1 = (r0 + c->Bq < Lq) ? r0 + c->Bq : Lq;
    const int nr = r1 - r0;
    const double* qs = c->q + (size_t)c->qoff[b] * Hq * d;
    const double* ks = c->k + (size_t)c->koff[b] * Hkv * d;
    const double* vs = c->v + (size_t)c->koff[b] * Hkv * d;
    double* os = c->o + (size_t)c->qoff[b] * Hq * d;
    const size_t srow = (size_t)c->lseoff[b] + (size_t)h * c->lse_hstride;
    double* buf = (double*)malloc(sizeof(double) * ((size_t)nr * (8 + d) + (size_t)nr * Bk));
    int32_t* slots = (int32_t*)calloc((size_t)nr, sizeof(int32_t));
    if (!buf || !slots) { free(buf); free(slots); return OR_ENOMEM; }
    double* m = buf;              /* running max of retained scores          */
    double* l = m + nr;           /* retained mass, shifted by m             */
    double* om = l + nr;          /* running max of omitted scores           */
    double* ol = om + nr;         /* omitted mass, shifted by om             */
    double* M = ol + nr;          /* tile row max                            */
    double* th = M + nr;          /* theta_i                                 */
    double* spare = th + nr;      /* (2 unused slots per row)                */
    double* acc = spare + 2 * (size_t)nr;   /* [nr][d] output accumulator    */
    double* S = acc + (size_t)nr * d;       /* [nr][Bk] tile scores          */
    for (int r = 0; r < nr; ++r) {
        m[r] = -INFINITY; l[r] = 0.0; om[r] = -INFINITY; ol[r] = 0.0;
        th[r] = log_threshold(c->tau, (double)(off + r0 + r + 1));   /* L_i = visible keys */
    }
    memset(acc, 0, sizeof(double) * (size_t)nr * d);

    /* tile holding the last legal key of the block's last row */
    const int kt_first = (off + r1 - 1) / Bk;
    for (int kt = kt_first; kt >= 0; --kt) {          /* diagonal -> earlier keys */
        const int j0 = kt * Bk;
        const int j1 = (j0 + Bk < Lk) ? j0 + Bk : Lk;
        /* score discovery: every legal key of the tile is scored */
        for (int r = 0; r < nr; ++r) {
            const int jl = off + r0 + r;              /* last key row r may see */
            const double* qi = qs + ((size_t)(r0 + r) * Hq + h) * d;
            double mx = -INFINITY;
            for (int j = j0; j < j1; ++j) {
                double s = -INFINITY;
                if (j <= jl) {
                    const double* kj = ks + ((size_t)j * Hkv + kh) * d;
                    s = dot(qi, kj, d) * c->scale;
                    if (s > mx) mx = s;
                }
                S[(size_t)r * Bk + (j - j0)] = s;
            }
            M[r] = mx;
        }
        /* decision: keep iff some valid row's ratio reaches tau / L_i */
        double lam = -INFINITY;
        for (int r = 0; r < nr; ++r) {
            if (M[r] == -INFINITY) continue;          /* no legal key: no vote */
            double x;
            if (l[r] == 0.0) x = INFINITY;            /* empty retained mass    */
            else x = M[r] - m[r] - log(l[r]) - th[r];
            if (x > lam) lam = x;
        }
        const int keep = (lam >= 0.0);
        const size_t tidx = (((size_t)b * Hq + h) * c->nQB + qb) * c->nKT + kt;
        if (c->keep) c->keep[tidx] = (uint8_t)keep;
        if (c->margin) c->margin[tidx] = lam;
        /* the decision the state update follows: the rule's, or a forced one */
        const int use = (c->forced && c->forced[tidx] != 255) ? (c->forced[tidx] != 0) : keep;

        for (int r = 0; r < nr; ++r) {
            if (M[r] == -INFINITY) continue;
            const int jl = off + r0 + r;
            const int nleg = ((jl < j1 - 1) ? jl : j1 - 1) - j0 + 1;
            if (use) {
                /* standard online-softmax update with the tile's legal keys */
                const double mn = (M[r] > m[r]) ? M[r] : m[r];
                const double alpha = (m[r] == -INFINITY) ? 0.0 : exp(m[r] - mn);
                double* ar = acc + (size_t)r * d;
                for (int cc = 0; cc < d; ++cc) ar[cc] *= alpha;
                double lsum = l[r] * alpha;
                for (int j = j0; j <= jl && j < j1; ++j) {
                    const double p = exp(S[(size_t)r * Bk + (j - j0)] - mn);
                    lsum += p;
                    const double* vj = vs + ((size_t)j * Hkv + kh) * d;
                    for (int cc = 0; cc < d; ++cc) ar[cc] += p * vj[cc];
                }
                l[r] = lsum;
                m[r] = mn;
                slots[r] += nleg;
            } else {
                /* bookkeeping only: mass of the omitted legal keys */
                const double mn = (M[r] > om[r]) ? M[r] : om[r];
                double osum = (om[r] == -INFINITY) ? 0.0 : ol[r] * exp(om[r] - mn);
                for (int j = j0; j <= jl && j < j1; ++j) osum += exp(S[(size_t)r * Bk + (j - j0)] - mn);
                ol[r] = osum;
                om[r] = mn;
            }
        }
    }
    for (int r = 0; r < nr; ++r) {
        const int i = r0 + r;
        const size_t orow = ((size_t)i * Hq + h) * d;
        for (int cc = 0; cc < d; ++cc) os[orow + cc] = acc[(size_t)r * d + cc] / l[r];
        const double lz = m[r] + log(l[r]);
        c->lse[srow + i] = lz;
        if (c->kept_slots) c->kept_slots[srow + i] = slots[r];
        if (c->omitted) {
            double w = 0.0;
            if (ol[r] > 0.0) w = 1.0 / (1.0 + exp(lz - (om[r] + log(ol[r]))));
            c->omitted[srow + i] = w;
        }
    }
    free(buf);
    free(slots);
    return OR_OK;
}

/* Runs the listed blocks (ids (b*Hq + h)*nQB + qb), or all of them longest
 * first when blocks is NULL. */
static int fwd_run(const fwd_ctx* c, const int32_t* blocks, int nblocks, int nthreads) {
    const int B = c->B, Hq = c->Hq;
    const long total = (long)B * Hq * c->nQB;
    const long n = blocks ? nblocks : total;
    int err = OR_OK;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < n; ++u) {
        long id = blocks ? (long)blocks[u] : u;
        if (id < 0 || id >= total) { err = OR_EINVAL; continue; }
        if (!blocks) {
            const long bh = id % ((long)B * Hq);
            const long qb = c->nQB - 1 - id / ((long)B * Hq);
            id = bh * c->nQB + qb;
        }
        const int qb = (int)(id % c->nQB);
        const int bh = (int)(id / c->nQB);
        int e = fwd_block(c, bh / Hq, bh % Hq, qb);
        if (e) err = e;
    }
    return err;
}

static int fwd_fixed(const double* q, const double* k, const double* v,
                     int B, int L, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                     const int32_t* blocks, int nblocks, const uint8_t* forced,
                     double* o, double* lse, uint8_t* keep, double* margin,
                     int32_t* kept_slots, double* omitted, int nthreads) {
    if (!q || !k || !v || !o || !lse) return OR_EINVAL;
    if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Bq <= 0 || Bk <= 0) return OR_EINVAL;
    if (Hq % Hkv != 0 || !tau_valid(tau)) return OR_EINVAL;
    long* offs = (long*)malloc(sizeof(long) * 3 * (size_t)B);
    int* lens = (int*)malloc(sizeof(int) * (size_t)B);
    if (!offs || !lens) { free(offs); free(lens); return OR_ENOMEM; }
    for (int b = 0; b < B; ++b) {
        offs[b] = (long)b * L;                     /* q and k rows */
        offs[B + b] = (long)b * Hq * L;            /* lse [B][Hq][L] */
        lens[b] = L;
    }
    fwd_ctx c;
    c.q = q; c.k = k; c.v = v; c.B = B; c.Hq = Hq; c.Hkv = Hkv; c.d = d;
    c.Bq = Bq; c.Bk = Bk; c.nQB = (L + Bq - 1) / Bq; c.nKT = (L + Bk - 1) / Bk;
    c.qoff = offs; c.koff = offs; c.lseoff = offs + B; c.lq = lens; c.lk = lens;
    c.lse_hstride = L;
    c.tau = tau; c.scale = 1.0 / sqrt((double)d);
    c.o = o; c.lse = lse; c.keep = keep; c.margin = margin; c.kept_slots = kept_slots; c.omitted = omitted;
    c.forced = forced;
    const int err = fwd_run(&c, blocks, nblocks, nthreads);
    free(offs);
    free(lens);
    return err;
}

int mala_oracle_fwd(const double* q, const double* k, const double* v,
                    int B, int L, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                    const int32_t* blocks, int nblocks,
                    double* o, double* lse, uint8_t* keep, double* margin,
                    int32_t* kept_slots, double* omitted, int nthreads) {
    return fwd_fixed(q, k, v, B, L, Hq, Hkv, d, tau, Bq, Bk, blocks, nblocks, NULL, o, lse, keep, margin,
                     kept_slots, omitted, nthreads);
}

/* Teacher-forced replay of the forward: where forced[tile] is 0 or 1 the
 * tile's state update follows that decision instead of the rule's, so the
 * rows' retained state is the one a run that took those decisions has.
 * keep and margin still record the rule's own decision and margin for every
 * tile, given that state.  With forced = the decisions of another
 * implementation, each of its decisions is judged from the state it had
 * itself: a decision that disagrees with the rule there is a genuine
 * difference (inside or outside the near-tie band), not a consequence of an
 * earlier one.  O, LSE and the statistics are those of the forced run. */
int mala_oracle_fwd_forced(const double* q, const double* k, const double* v,
                           int B, int L, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                           const int32_t* blocks, int nblocks, const uint8_t* forced,
                           double* o, double* lse, uint8_t* keep, double* margin,
                           int32_t* kept_slots, double* omitted, int nthreads) {
    if (!forced) return OR_EINVAL;
    return fwd_fixed(q, k, v, B, L, Hq, Hkv, d, tau, Bq, Bk, blocks, nblocks, forced, o, lse, keep, margin,
                     kept_slots, omitted, nthreads);
}

/* Variable-length forward: sequence b has queries cu_q[b] .. cu_q[b+1]-1 and
 * keys cu_k[b] .. cu_k[b+1]-1 of the packed arrays, with its queries at the
 * end of its keys (0 <= Lq <= Lk).  Layouts in the header comment; nQB and
 * nKT from the longest query and key lengths. */
static int fwd_varlen_impl(const double* q, const double* k, const double* v,
                           const int32_t* cu_q, const int32_t* cu_k,
                           int B, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                           const int32_t* blocks, int nblocks, const uint8_t* forced,
                           double* o, double* lse, uint8_t* keep, double* margin,
                           int32_t* kept_slots, double* omitted, int nthreads) {
    if (!q || !k || !v || !o || !lse || !cu_q || !cu_k) return OR_EINVAL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Bq <= 0 || Bk <= 0) return OR_EINVAL;
    if (Hq % Hkv != 0 || !tau_valid(tau)) return OR_EINVAL;
    if (cu_q[0] != 0 || cu_k[0] != 0) return OR_EINVAL;
    int maxq = 0, maxk = 0;
    for (int b = 0; b < B; ++b) {
        const int lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
        if (lq < 0 || lk < lq) return OR_EINVAL;
        if (lq > maxq) maxq = lq;
        if (lk > maxk) maxk = lk;
    }
    long* offs = (long*)malloc(sizeof(long) * 3 * (size_t)B);
    int* lens = (int*)malloc(sizeof(int) * 2 * (size_t)B);
    if (!offs || !lens) { free(offs); free(lens); return OR_ENOMEM; }
    for (int b = 0; b < B; ++b) {
        offs[b] = cu_q[b];
        offs[B + b] = cu_k[b];
        offs[2 * B + b] = cu_q[b];                 /* lse [Hq][total_q] */
        lens[b] = cu_q[b + 1] - cu_q[b];
        lens[B + b] = cu_k[b + 1] - cu_k[b];
    }
    fwd_ctx c;
    c.q = q; c.k = k; c.v = v; c.B = B; c.Hq = Hq; c.Hkv = Hkv; c.d = d;
    c.Bq = Bq; c.Bk = Bk;
    c.nQB = maxq > 0 ? (maxq + Bq - 1) / Bq : 1;
    c.nKT = maxk > 0 ? (maxk + Bk - 1) / Bk : 1;
    c.qoff = offs; c.koff = offs + B; c.lseoff = offs + 2 * B; c.lq = lens; c.lk = lens + B;
    c.lse_hstride = cu_q[B];
    c.tau = tau; c.scale = 1.0 / sqrt((double)d);
    c.o = o; c.lse = lse; c.keep = keep; c.margin = margin; c.kept_slots = kept_slots; c.omitted = omitted;
    c.forced = forced;
    const int err = fwd_run(&c, blocks, nblocks, nthreads);
    free(offs);
    free(lens);
    return err;
}

int mala_oracle_fwd_varlen(const double* q, const double* k, const double* v,
                           const int32_t* cu_q, const int32_t* cu_k,
                           int B, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                           const int32_t* blocks, int nblocks,
                           double* o, double* lse, uint8_t* keep, double* margin,
                           int32_t* kept_slots, double* omitted, int nthreads) {
    return fwd_varlen_impl(q, k, v, cu_q, cu_k, B, Hq, Hkv, d, tau, Bq, Bk, blocks, nblocks, NULL, o, lse, keep,
                           margin, kept_slots, omitted, nthreads);
}

/* Teacher-forced replay of the variable-length forward, as
 * mala_oracle_fwd_forced (forced has keep's layout, [B][Hq][nQB][nKT]). */
int mala_oracle_fwd_varlen_forced(const double* q, const double* k, const double* v,
                                  const int32_t* cu_q, const int32_t* cu_k,
                                  int B, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                                  const int32_t* blocks, int nblocks, const uint8_t* forced,
                                  double* o, double* lse, uint8_t* keep, double* margin,
                                  int32_t* kept_slots, double* omitted, int nthreads) {
    if (!forced) return OR_EINVAL;
    return fwd_varlen_impl(q, k, v, cu_q, cu_k, B, Hq, Hkv, d, tau, Bq, Bk, blocks, nblocks, forced, o, lse, keep,
                           margin, kept_slots, omitted, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Backward ([P2] "Backward: offline sparse probabilities"; [P1] backward)  */
/* ------------------------------------------------------------------------ */
typedef struct {
    const double *q, *k, *v, *o, *dout, *lse;
    int B, Hq, Hkv, d, Bq, Bk, nQB, nKT;
    /* per sequence, as in fwd_ctx */
    const long *qoff, *koff, *lseoff;
    const int *lq, *lk;
    long lse_hstride;
    double tau, scale;
    double *dq, *dk, *dv, *margin;
    double *dq_cond, *dk_cond;   /* NULL = not computed */
    uint8_t* keep;
} bwd_ctx;

/* Row i of sequence b in a [rows][H][d] array, and its lse entry for head h. */
static size_t qrow(const bwd_ctx* c, int b, int i, int h) {
    return (((size_t)c->qoff[b] + i) * c->Hq + h) * c->d;
}
static size_t krow(const bwd_ctx* c, int b, int j, int kh) {
    return (((size_t)c->koff[b] + j) * c->Hkv + kh) * c->d;
}
static double lse_at(const bwd_ctx* c, int b, int h, int i) {
    return c->lse[(size_t)c->lseoff[b] + (size_t)h * c->lse_hstride + i];
}

/* Scores of tile (qb, kt) for q head h and the offline decision.  S is
 * [nr][Bk] with -inf on illegal entries.  Returns keep (0/1). */
static int bwd_tile(const bwd_ctx* c, int b, int h, int qb, int kt, double* S, double* lam_out) {
    const int d = c->d, Hq = c->Hq, Hkv = c->Hkv, Bk = c->Bk;
    const int Lq = c->lq[b], Lk = c->lk[b], off = Lk - Lq;
    const int kh = h / (Hq / Hkv);
    const int r0 = qb * c->Bq;
    const int r1 = (r0 + c->Bq < Lq) ? r0 + c->Bq : Lq;
    const int j0 = kt * Bk;
    const int j1 = (j0 + Bk < Lk) ? j0 + Bk : Lk;
    double lam = -INFINITY;
    for (int i = r0; i < r1; ++i) {
        const double* qi = c->q + qrow(c, b, i, h);
        const double lz = lse_at(c, b, h, i);
        const double th = log_threshold(c->tau, (double)(off + i + 1));
        double mx = -INFINITY;
        for (int j = j0; j < j1; ++j) {
            double s = -INFINITY;
            if (j <= off + i) {
                s = dot(qi, c->k + krow(c, b, j, kh), d) * c->scale;
                if (s > mx) mx = s;
            }
            S[(size_t)(i - r0) * Bk + (j - j0)] = s;
        }
        if (mx == -INFINITY) continue;
        const double x = mx - lz - th;
        if (x > lam) lam = x;
    }
    *lam_out = lam;
    return lam >= 0.0;
}

static void record_bwd(const bwd_ctx* c, int b, int h, int qb, int kt, int keep, double lam) {
    const size_t tidx = (((size_t)b * c->Hq + h) * c->nQB + qb) * c->nKT + kt;
    if (c->keep) c->keep[tidx] = (uint8_t)keep;
    if (c->margin) c->margin[tidx] = lam;
}

/* dq for one query block: sum over its kept tiles. */
static int bwd_dq_block(const bwd_ctx* c, int b, int h, int qb) {
    const int d = c->d, Hq = c->Hq, Hkv = c->Hkv, Bk = c->Bk;
    const int Lq = c->lq[b], Lk = c->lk[b], off = Lk - Lq;
    const int kh = h / (Hq / Hkv);
    const int r0 = qb * c->Bq;
    if (r0 >= Lq) return OR_OK;                /* past the sequence's queries */
    const int r1 = (r0 + c->Bq < Lq) ? r0 + c->Bq : Lq;
    const int nr = r1 - r0;
    double* S = (double*)malloc(sizeof(double) * ((size_t)nr * Bk + 2 * (size_t)nr));
    if (!S) return OR_ENOMEM;
    double* D = S + (size_t)nr * Bk;
    double* Da = D + nr;          /* |dO_i|.|o_i|, for dq_cond */
    for (int i = r0; i < r1; ++i) {
        const size_t row = qrow(c, b, i, h);
        D[i - r0] = dot(c->dout + row, c->o + row, d);
        Da[i - r0] = dot_abs(c->dout + row, c->o + row, d);
        for (int cc = 0; cc < d; ++cc) c->dq[row + cc] = 0.0;
        if (c->dq_cond)
            for (int cc = 0; cc < d; ++cc) c->dq_cond[row + cc] = 0.0;
    }
    const int kt_last = (off + r1 - 1) / Bk;
    for (int kt = 0; kt <= kt_last; ++kt) {
        double lam;
        const int keep = bwd_tile(c, b, h, qb, kt, S, &lam);
        record_bwd(c, b, h, qb, kt, keep, lam);
        if (!keep) continue;
        const int j0 = kt * Bk;
        const int j1 = (j0 + Bk < Lk) ? j0 + Bk : Lk;
        for (int i = r0; i < r1; ++i) {
            const size_t row = qrow(c, b, i, h);
            const double lz = lse_at(c, b, h, i);
            for (int j = j0; j < j1 && j <= off + i; ++j) {
                const double* vj = c->v + krow(c, b, j, kh);
                const double* kj = c->k + krow(c, b, j, kh);
                const double p = exp(S[(size_t)(i - r0) * Bk + (j - j0)] - lz);
                const double dp = dot(c->dout + row, vj, d);
                const double ds = p * (dp - D[i - r0]);
                for (int cc = 0; cc < d; ++cc) c->dq[row + cc] += c->scale * ds * kj[cc];
                if (c->dq_cond) {
                    const double w = p * (dot_abs(c->dout + row, vj, d) + Da[i - r0]);
                    for (int cc = 0; cc < d; ++cc) c->dq_cond[row + cc] += c->scale * w * fabs(kj[cc]);
                }
            }
        }
    }
    free(S);
    return OR_OK;
}

/* dk, dv for one key tile of one KV head: sum over the q heads of the group
 * and over every query block that can see the tile. */
static int bwd_dkdv_tile(const bwd_ctx* c, int b, int kh, int kt) {
    const int d = c->d, Hq = c->Hq, Hkv = c->Hkv, Bk = c->Bk, Bq = c->Bq;
    const int Lq = c->lq[b], Lk = c->lk[b], off = Lk - Lq;
    const int G = Hq / Hkv;
    const int j0 = kt * Bk;
    if (j0 >= Lk) return OR_OK;                /* past the sequence's keys */
    const int j1 = (j0 + Bk < Lk) ? j0 + Bk : Lk;
    const int nQBb = (Lq + Bq - 1) / Bq;
    const int qb_lo = (j0 - off > 0 ? j0 - off : 0) / Bq;   /* first block with a row seeing key j0 */
    double* S = (double*)malloc(sizeof(double) * ((size_t)Bq * Bk + 2 * (size_t)Bq));
    if (!S) return OR_ENOMEM;
    double* D = S + (size_t)Bq * Bk;
    double* Da = D + Bq;          /* |dO_i|.|o_i|, for dk_cond */
    for (int j = j0; j < j1; ++j) {
        const size_t kr = krow(c, b, j, kh);
        for (int cc = 0; cc < d; ++cc) { c->dk[kr + cc] = 0.0; c->dv[kr + cc] = 0.0; }
        if (c->dk_cond)
            for (int cc = 0; cc < d; ++cc) c->dk_cond[kr + cc] = 0.0;
    }
    for (int g = 0; g < G; ++g) {
        const int h = kh * G + g;
        for (int qb = qb_lo; qb < nQBb; ++qb) {
            const int r0 = qb * Bq;
            const int r1 = (r0 + Bq < Lq) ? r0 + Bq : Lq;
            double lam;
            const int keep = bwd_tile(c, b, h, qb, kt, S, &lam);
            record_bwd(c, b, h, qb, kt, keep, lam);
            if (!keep) continue;
            for (int i = r0; i < r1; ++i) {
                const size_t row = qrow(c, b, i, h);
                D[i - r0] = dot(c->dout + row, c->o + row, d);
                Da[i - r0] = dot_abs(c->dout + row, c->o + row, d);
            }
            for (int i = r0; i < r1; ++i) {
                const size_t row = qrow(c, b, i, h);
                const double lz = lse_at(c, b, h, i);
                for (int j = j0; j < j1 && j <= off + i; ++j) {
                    const size_t kr = krow(c, b, j, kh);
                    const double p = exp(S[(size_t)(i - r0) * Bk + (j - j0)] - lz);
                    const double dp = dot(c->dout + row, c->v + kr, d);
                    const double ds = p * (dp - D[i - r0]);
                    for (int cc = 0; cc < d; ++cc) {
                        c->dv[kr + cc] += p * c->dout[row + cc];
                        c->dk[kr + cc] += c->scale * ds * c->q[row + cc];
                    }
                    if (c->dk_cond) {
                        const double w = p * (dot_abs(c->dout + row, c->v + kr, d) + Da[i - r0]);
                        for (int cc = 0; cc < d; ++cc) c->dk_cond[kr + cc] += c->scale * w * fabs(c->q[row + cc]);
                    }
                }
            }
        }
    }
    free(S);
    return OR_OK;
}

/* qunits: ids (b*Hq + h)*nQB + qb whose dq rows are computed (NULL: all).
 * kunits: ids (b*Hkv + kh)*nKT + kt whose dk/dv rows are computed (NULL: all).
 * nq / nk < 0 with a NULL list skips that pass entirely. */
static int bwd_run(const bwd_ctx* c, const int32_t* qunits, int nq, const int32_t* kunits, int nk, int nthreads) {
    const int B = c->B, Hq = c->Hq, Hkv = c->Hkv;
    int err = OR_OK;
    set_threads(nthreads);
    const long totq = (long)B * Hq * c->nQB;
    const long nqq = qunits ? nq : (nq < 0 ? 0 : totq);
    if (nqq > 0 && !c->dq) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < nqq; ++u) {
        long id = qunits ? (long)qunits[u] : u;
        if (id < 0 || id >= totq) { err = OR_EINVAL; continue; }
        const int qb = (int)(id % c->nQB);
        const int bh = (int)(id / c->nQB);
        int e = bwd_dq_block(c, bh / Hq, bh % Hq, qb);
        if (e) err = e;
    }
    const long totk = (long)B * Hkv * c->nKT;
    const long nkk = kunits ? nk : (nk < 0 ? 0 : totk);
    if (nkk > 0 && (!c->dk || !c->dv)) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < nkk; ++u) {
        long id = kunits ? (long)kunits[u] : u;
        if (id < 0 || id >= totk) { err = OR_EINVAL; continue; }
        const int kt = (int)(id % c->nKT);
        const int bk = (int)(id / c->nKT);
        int e = bwd_dkdv_tile(c, bk / Hkv, bk % Hkv, kt);
        if (e) err = e;
    }
    return err;
}

int mala_oracle_bwd(const double* q, const double* k, const double* v, const double* o,
                    const double* dout, const double* lse,
                    int B, int L, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                    const int32_t* qunits, int nq, const int32_t* kunits, int nk,
                    double* dq, double* dk, double* dv, uint8_t* keep, double* margin,
                    double* dq_cond, double* dk_cond, int nthreads) {
    if (!q || !k || !v || !o || !dout || !lse) return OR_EINVAL;
    if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Bq <= 0 || Bk <= 0) return OR_EINVAL;
    if (Hq % Hkv != 0 || !tau_valid(tau)) return OR_EINVAL;
    long* offs = (long*)malloc(sizeof(long) * 2 * (size_t)B);
    int* lens = (int*)malloc(sizeof(int) * (size_t)B);
    if (!offs || !lens) { free(offs); free(lens); return OR_ENOMEM; }
    for (int b = 0; b < B; ++b) {
        offs[b] = (long)b * L;
        offs[B + b] = (long)b * Hq * L;
        lens[b] = L;
    }
    bwd_ctx c;
    c.q = q; c.k = k; c.v = v; c.o = o; c.dout = dout; c.lse = lse;
    c.B = B; c.Hq = Hq; c.Hkv = Hkv; c.d = d; c.Bq = Bq; c.Bk = Bk;
    c.nQB = (L + Bq - 1) / Bq; c.nKT = (L + Bk - 1) / Bk;
    c.qoff = offs; c.koff = offs; c.lseoff = offs + B; c.lq = lens; c.lk = lens; c.lse_hstride = L;
    c.tau = tau; c.scale = 1.0 / sqrt((double)d);
    c.dq = dq; c.dk = dk; c.dv = dv; c.keep = keep; c.margin = margin;
    c.dq_cond = dq_cond; c.dk_cond = dk_cond;
    const int err = bwd_run(&c, qunits, nq, kunits, nk, nthreads);
    free(offs);
    free(lens);
    return err;
}

/* Variable-length backward over the packed layout of mala_oracle_fwd_varlen:
 * q, o, dout, dq [total_q][Hq][d]; k, v, dk, dv [total_k][Hkv][d]; lse
 * [Hq][total_q]; keep/margin [B][Hq][nQB][nKT] with nQB, nKT from the longest
 * query and key lengths.  Keys of a sequence without queries get dk = dv = 0. */
int mala_oracle_bwd_varlen(const double* q, const double* k, const double* v, const double* o,
                           const double* dout, const double* lse, const int32_t* cu_q, const int32_t* cu_k,
                           int B, int Hq, int Hkv, int d, double tau, int Bq, int Bk,
                           const int32_t* qunits, int nq, const int32_t* kunits, int nk,
                           double* dq, double* dk, double* dv, uint8_t* keep, double* margin,
                           double* dq_cond, double* dk_cond, int nthreads) {
    if (!q || !k || !v || !o || !dout || !lse || !cu_q || !cu_k) return OR_EINVAL;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Bq <= 0 || Bk <= 0) return OR_EINVAL;
    if (Hq % Hkv != 0 || !tau_valid(tau)) return OR_EINVAL;
    if (cu_q[0] != 0 || cu_k[0] != 0) return OR_EINVAL;
    int maxq = 0, maxk = 0;
    for (int b = 0; b < B; ++b) {
        const int lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
        if (lq < 0 || lk < lq) return OR_EINVAL;
        if (lq > maxq) maxq = lq;
        if (lk > maxk) maxk = lk;
    }
    long* offs = (long*)malloc(sizeof(long) * 3 * (size_t)B);
    int* lens = (int*)malloc(sizeof(int) * 2 * (size_t)B);
    if (!offs || !lens) { free(offs); free(lens); return OR_ENOMEM; }
    for (int b = 0; b < B; ++b) {
        offs[b] = cu_q[b];
        offs[B + b] = cu_k[b];
        offs[2 * B + b] = cu_q[b];
        lens[b] = cu_q[b + 1] - cu_q[b];
        lens[B + b] = cu_k[b + 1] - cu_k[b];
    }
    bwd_ctx c;
    c.q = q; c.k = k; c.v = v; c.o = o; c.dout = dout; c.lse = lse;
    c.B = B; c.Hq = Hq; c.Hkv = Hkv; c.d = d; c.Bq = Bq; c.Bk = Bk;
    c.nQB = maxq > 0 ? (maxq + Bq - 1) / Bq : 1;
    c.nKT = maxk > 0 ? (maxk + Bk - 1) / Bk : 1;
    c.qoff = offs; c.koff = offs + B; c.lseoff = offs + 2 * B; c.lq = lens; c.lk = lens + B;
    c.lse_hstride = cu_q[B];
    c.tau = tau; c.scale = 1.0 / sqrt((double)d);
    c.dq = dq; c.dk = dk; c.dv = dv; c.keep = keep; c.margin = margin;
    c.dq_cond = dq_cond; c.dk_cond = dk_cond;
    const int err = bwd_run(&c, qunits, nq, kunits, nk, nthreads);
    free(offs);
    free(lens);
    return err;
}

/* ------------------------------------------------------------------------ */
/* Decode: the forward rule for one new token against a cache of N keys.    */
/* Rows of a decision are the G q heads sharing a KV head; L_i = N.          */
/* q, o: [B][Hq][d]; kc, vc: [B][N][Hkv][d]; lse, omitted: [B][Hq];          */
/* keep, margin: [B][Hkv][nT] with nT = ceil(N/Bkd); kept_tiles: [B][Hkv].   */
/* seqlens: NULL, or [B] cache lengths 1 <= N_b <= N: sequence b then uses   */
/* its first N_b cache rows, with L_i = N_b and tiles 0 .. ceil(N_b/Bkd)-1   */
/* (entries of later tiles are not written).                                 */
/* ------------------------------------------------------------------------ */
static int decode_impl(const double* q, const double* kc, const double* vc,
                       int B, int N, int Hq, int Hkv, int d, double tau, int Bkd,
                       const int32_t* seqlens, const uint8_t* forced,
                       double* o, double* lse, uint8_t* keep, double* margin,
                       int32_t* kept_tiles, double* omitted, int nthreads) {
    if (!q || !kc || !vc || !o || !lse) return OR_EINVAL;
    if (B <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Bkd <= 0) return OR_EINVAL;
    if (Hq % Hkv != 0 || !tau_valid(tau)) return OR_EINVAL;
    if (seqlens)
        for (int b = 0; b < B; ++b)
            if (seqlens[b] < 1 || seqlens[b] > N) return OR_EINVAL;
    const int G = Hq / Hkv;
    const int nTmax = (N + Bkd - 1) / Bkd;     /* stride of keep / margin */
    const double scale = 1.0 / sqrt((double)d);
    int err = OR_OK;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < (long)B * Hkv; ++u) {
        const int b = (int)(u / Hkv), kh = (int)(u % Hkv);
        const int Nb = seqlens ? seqlens[b] : N;          /* this sequence's keys */
        const int nT = (Nb + Bkd - 1) / Bkd;
        const double th = log_threshold(tau, (double)Nb);
        double* buf = (double*)malloc(sizeof(double) * ((size_t)G * (5 + d) + (size_t)G * Bkd));
        if (!buf) { err = OR_ENOMEM; continue; }
        double *m = buf, *l = m + G, *om = l + G, *ol = om + G, *M = ol + G;
        double* acc = M + G;
        double* S = acc + (size_t)G * d;
        for (int g = 0; g < G; ++g) { m[g] = -INFINITY; l[g] = 0.0; om[g] = -INFINITY; ol[g] = 0.0; }
        memset(acc, 0, sizeof(double) * (size_t)G * d);
        int nkept = 0;
        for (int t = nT - 1; t >= 0; --t) {            /* newest tile first */
            const int j0 = t * Bkd;
            const int j1 = (j0 + Bkd < Nb) ? j0 + Bkd : Nb;
            double lam = -INFINITY;
            for (int g = 0; g < G; ++g) {
                const double* qg = q + ((size_t)b * Hq + kh * G + g) * d;
                double mx = -INFINITY;
                for (int j = j0; j < j1; ++j) {
                    const double s = dot(qg, kc + (((size_t)b * N + j) * Hkv + kh) * d, d) * scale;
                    S[(size_t)g * Bkd + (j - j0)] = s;
                    if (s > mx) mx = s;
                }
                M[g] = mx;
                const double x = (l[g] == 0.0) ? INFINITY : mx - m[g] - log(l[g]) - th;
                if (x > lam) lam = x;
            }
            const size_t tidx = ((size_t)b * Hkv + kh) * nTmax + t;
            const int own = (lam >= 0.0);
            if (keep) keep[tidx] = (uint8_t)own;
            if (margin) margin[tidx] = lam;
            /* the decision the state update follows: the rule's, or a forced one */
            const int kp = (forced && forced[tidx] != 255) ? (forced[tidx] != 0) : own;
            nkept += kp;
            for (int g = 0; g < G; ++g) {
                if (kp) {
                    const double mn = (M[g] > m[g]) ? M[g] : m[g];
                    const double alpha = (m[g] == -INFINITY) ? 0.0 : exp(m[g] - mn);
                    double* ar = acc + (size_t)g * d;
                    for (int cc = 0; cc < d; ++cc) ar[cc] *= alpha;
                    double lsum = l[g] * alpha;
                    for (int j = j0; j < j1; ++j) {
                        const double p = exp(S[(size_t)g * Bkd + (j - j0)] - mn);
                        lsum += p;
                        const double* vj = vc + (((size_t)b * N + j) * Hkv + kh) * d;
                        for (int cc = 0; cc < d; ++cc) ar[cc] += p * vj[cc];
                    }
                    l[g] = lsum;
                    m[g] = mn;
                } else {
                    const double mn = (M[g] > om[g]) ? M[g] : om[g];
                    double osum = (om[g] == -INFINITY) ? 0.0 : ol[g] * exp(om[g] - mn);
                    for (int j = j0; j < j1; ++j) osum += exp(S[(size_t)g * Bkd + (j - j0)] - mn);
                    ol[g] = osum;
                    om[g] = mn;
                }
            }
        }
        for (int g = 0; g < G; ++g) {
            const int h = kh * G + g;
            for (int cc = 0; cc < d; ++cc) o[((size_t)b * Hq + h) * d + cc] = acc[(size_t)g * d + cc] / l[g];
            const double lz = m[g] + log(l[g]);
            lse[(size_t)b * Hq + h] = lz;
            if (omitted) {
                double w = 0.0;
                if (ol[g] > 0.0) w = 1.0 / (1.0 + exp(lz - (om[g] + log(ol[g]))));
                omitted[(size_t)b * Hq + h] = w;
            }
        }
        if (kept_tiles) kept_tiles[(size_t)b * Hkv + kh] = nkept;
        free(buf);
    }
    return err;
}

int mala_oracle_decode(const double* q, const double* kc, const double* vc,
                       int B, int N, int Hq, int Hkv, int d, double tau, int Bkd,
                       const int32_t* seqlens,
                       double* o, double* lse, uint8_t* keep, double* margin,
                       int32_t* kept_tiles, double* omitted, int nthreads) {
    return decode_impl(q, kc, vc, B, N, Hq, Hkv, d, tau, Bkd, seqlens, NULL, o, lse, keep, margin, kept_tiles,
                       omitted, nthreads);
}

/* Teacher-forced replay of the decode rule, as mala_oracle_fwd_forced:
 * forced is [B][Hkv][nT] (0 / 1 forces the decision the update follows, 255
 * leaves it to the rule); keep and margin record the rule's own decision and
 * margin given that state; kept_tiles counts the decisions followed. */
int mala_oracle_decode_forced(const double* q, const double* kc, const double* vc,
                              int B, int N, int Hq, int Hkv, int d, double tau, int Bkd,
                              const int32_t* seqlens, const uint8_t* forced,
                              double* o, double* lse, uint8_t* keep, double* margin,
                              int32_t* kept_tiles, double* omitted, int nthreads) {
    if (!forced) return OR_EINVAL;
    return decode_impl(q, kc, vc, B, N, Hq, Hkv, d, tau, Bkd, seqlens, forced, o, lse, keep, margin, kept_tiles,
                       omitted, nthreads);
}
