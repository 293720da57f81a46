/*
 * Drives every entry point of the fp64 oracle (oracle/mala_oracle.c) on small
 * ragged shapes, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer checks its index arithmetic: block and tile
 * bounds, packed sequence offsets, unit lists, cache lengths.  Test
 * infrastructure only (tests/test_oracle_sanitized.py builds and runs it on the
 * CPU).  Exit status 0 = every call returned OK and every output is sane.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int mala_oracle_fwd(const double*, const double*, const double*, int, int, int, int, int, double, int, int,
                    const int32_t*, int, double*, double*, uint8_t*, double*, int32_t*, double*, int);
int mala_oracle_bwd(const double*, const double*, const double*, const double*, const double*, const double*,
                    int, int, int, int, int, double, int, int, const int32_t*, int, const int32_t*, int,
                    double*, double*, double*, uint8_t*, double*, double*, double*, int);
int mala_oracle_fwd_varlen(const double*, const double*, const double*, const int32_t*, const int32_t*, int, int,
                           int, int, double, int, int, const int32_t*, int, double*, double*, uint8_t*, double*,
                           int32_t*, double*, int);
int mala_oracle_bwd_varlen(const double*, const double*, const double*, const double*, const double*,
                           const double*, const int32_t*, const int32_t*, int, int, int, int, double, int, int,
                           const int32_t*, int, const int32_t*, int, double*, double*, double*, uint8_t*, double*,
                           double*, double*, int);
int mala_oracle_decode(const double*, const double*, const double*, int, int, int, int, int, double, int,
                       const int32_t*, double*, double*, uint8_t*, double*, int32_t*, double*, int);
int mala_oracle_fwd_forced(const double*, const double*, const double*, int, int, int, int, int, double, int, int,
                           const int32_t*, int, const uint8_t*, double*, double*, uint8_t*, double*, int32_t*,
                           double*, int);
int mala_oracle_fwd_varlen_forced(const double*, const double*, const double*, const int32_t*, const int32_t*, int,
                                  int, int, int, double, int, int, const int32_t*, int, const uint8_t*, double*,
                                  double*, uint8_t*, double*, int32_t*, double*, int);
int mala_oracle_decode_forced(const double*, const double*, const double*, int, int, int, int, int, double, int,
                              const int32_t*, const uint8_t*, double*, double*, uint8_t*, double*, int32_t*, double*,
                              int);

/* A teacher-forcing array from decisions: every third visited tile flipped,
 * the rest left to the rule (255). */
static uint8_t* flip_every_third(const uint8_t* keep, size_t n) {
    uint8_t* f = (uint8_t*)malloc(n ? n : 1);
    for (size_t i = 0; i < n; ++i) f[i] = (i % 3 == 0 && keep[i] <= 1) ? (uint8_t)(1 - keep[i]) : 255;
    return f;
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {   /* xorshift64*, uniform in [-1, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}

/* Exactly sized heap arrays, so any read or write past the end is caught. */
static double* darr(size_t n, int fill) {
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = fill ? 2.0 * urand() : 0.0;
    return p;
}

static int failures = 0;
#define CHECK(cond, what)                                              \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "FAIL %s (line %d)\n", what, __LINE__);    \
            ++failures;                                                \
        }                                                              \
    } while (0)

static void fixed_case(int B, int L, int Hq, int Hkv, int d, double tau, int Bq, int Bk, int sampled) {
    const size_t nq = (size_t)B * L * Hq * d, nk = (size_t)B * L * Hkv * d;
    const int nQB = (L + Bq - 1) / Bq, nKT = (L + Bk - 1) / Bk;
    const size_t nt = (size_t)B * Hq * nQB * nKT;
    double *q = darr(nq, 1), *k = darr(nk, 1), *v = darr(nk, 1), *dout = darr(nq, 1);
    double *o = darr(nq, 0), *lse = darr((size_t)B * Hq * L, 0), *margin = darr(nt, 0), *om = darr((size_t)B * Hq * L, 0);
    uint8_t* keep = (uint8_t*)calloc(nt, 1);
    int32_t* slots = (int32_t*)calloc((size_t)B * Hq * L, sizeof(int32_t));
    int32_t blocks[3] = {0, B * Hq * nQB - 1, (B * Hq * nQB) / 2};
    int rc = mala_oracle_fwd(q, k, v, B, L, Hq, Hkv, d, tau, Bq, Bk, sampled ? blocks : NULL, sampled ? 3 : 0,
                             o, lse, keep, margin, slots, om, 1);
    CHECK(rc == 0, "fwd rc");
    if (!sampled)
        for (size_t i = 0; i < nq; ++i) CHECK(isfinite(o[i]), "fwd o finite");
    {   /* teacher-forced replay over the same outputs */
        uint8_t* fz = flip_every_third(keep, nt);
        rc = mala_oracle_fwd_forced(q, k, v, B, L, Hq, Hkv, d, tau, Bq, Bk, sampled ? blocks : NULL, sampled ? 3 : 0,
                                    fz, o, lse, keep, margin, slots, om, 1);
        CHECK(rc == 0, "fwd_forced rc");
        CHECK(mala_oracle_fwd_forced(q, k, v, B, L, Hq, Hkv, d, tau, Bq, Bk, NULL, 0, NULL, o, lse, keep, margin,
                                     slots, om, 1) != 0, "fwd_forced refuses a NULL forcing array");
        free(fz);
        rc = mala_oracle_fwd(q, k, v, B, L, Hq, Hkv, d, tau, Bq, Bk, sampled ? blocks : NULL, sampled ? 3 : 0,
                             o, lse, keep, margin, slots, om, 1);   /* free-run outputs for the backward */
        CHECK(rc == 0, "fwd rc (again)");
    }
    double *dq = darr(nq, 0), *dk = darr(nk, 0), *dv = darr(nk, 0), *dqc = darr(nq, 0), *dkc = darr(nk, 0);
    int32_t kunits[2] = {0, B * Hkv * nKT - 1};
    rc = mala_oracle_bwd(q, k, v, o, dout, lse, B, L, Hq, Hkv, d, tau, Bq, Bk, sampled ? blocks : NULL,
                         sampled ? 3 : 0, sampled ? kunits : NULL, sampled ? 2 : 0, dq, dk, dv, keep, margin, dqc,
                         dkc, 1);
    CHECK(rc == 0, "bwd rc");
    for (size_t i = 0; i < nt; ++i) CHECK(keep[i] <= 1, "keep is 0/1");
    if (!sampled)
        for (size_t i = 0; i < nq; ++i) CHECK(isfinite(dq[i]) && dqc[i] >= 0.0, "bwd dq finite, cond >= 0");
    /* invalid calls are refused, not run */
    CHECK(mala_oracle_fwd(q, k, v, B, L, Hq, Hq + 1, d, tau, Bq, Bk, NULL, 0, o, lse, keep, margin, slots, om, 1) != 0,
          "fwd refuses Hq % Hkv != 0");
    CHECK(mala_oracle_fwd(q, k, v, B, L, Hq, Hkv, d, -1.0, Bq, Bk, NULL, 0, o, lse, keep, margin, slots, om, 1) != 0,
          "fwd refuses tau < 0");
    int32_t badblk[1] = {B * Hq * nQB};
    CHECK(mala_oracle_fwd(q, k, v, B, L, Hq, Hkv, d, tau, Bq, Bk, badblk, 1, o, lse, keep, margin, slots, om, 1) != 0,
          "fwd refuses a block id past the end");
    free(q); free(k); free(v); free(dout); free(o); free(lse); free(margin); free(om); free(keep); free(slots);
    free(dq); free(dk); free(dv); free(dqc); free(dkc);
}

static void varlen_case(int B, const int* lq, const int* lk, int Hq, int Hkv, int d, double tau, int Bq, int Bk) {
    int32_t* cq = (int32_t*)malloc(sizeof(int32_t) * (B + 1));
    int32_t* ck = (int32_t*)malloc(sizeof(int32_t) * (B + 1));
    cq[0] = ck[0] = 0;
    int maxq = 0, maxk = 0;
    for (int b = 0; b < B; ++b) {
        cq[b + 1] = cq[b] + lq[b];
        ck[b + 1] = ck[b] + lk[b];
        if (lq[b] > maxq) maxq = lq[b];
        if (lk[b] > maxk) maxk = lk[b];
    }
    const int Tq = cq[B], Tk = ck[B];
    const int nQB = maxq > 0 ? (maxq + Bq - 1) / Bq : 1, nKT = maxk > 0 ? (maxk + Bk - 1) / Bk : 1;
    const size_t nt = (size_t)B * Hq * nQB * nKT;
    const size_t nq = (size_t)Tq * Hq * d, nk = (size_t)Tk * Hkv * d;
    double *q = darr(nq, 1), *k = darr(nk, 1), *v = darr(nk, 1), *dout = darr(nq, 1);
    double *o = darr(nq, 0), *lse = darr((size_t)Hq * Tq, 0), *margin = darr(nt, 0), *om = darr((size_t)Hq * Tq, 0);
    uint8_t* keep = (uint8_t*)calloc(nt, 1);
    int32_t* slots = (int32_t*)calloc((size_t)Hq * Tq + 1, sizeof(int32_t));
    int rc = mala_oracle_fwd_varlen(q, k, v, cq, ck, B, Hq, Hkv, d, tau, Bq, Bk, NULL, 0, o, lse, keep, margin, slots,
                                    om, 1);
    CHECK(rc == 0, "fwd_varlen rc");
    {
        uint8_t* fz = flip_every_third(keep, nt);
        double *o2 = darr(nq, 0), *lse2 = darr((size_t)Hq * Tq, 0), *om2 = darr((size_t)Hq * Tq, 0);
        double* margin2 = darr(nt, 0);
        uint8_t* keep2 = (uint8_t*)calloc(nt, 1);
        int32_t* slots2 = (int32_t*)calloc((size_t)Hq * Tq + 1, sizeof(int32_t));
        CHECK(mala_oracle_fwd_varlen_forced(q, k, v, cq, ck, B, Hq, Hkv, d, tau, Bq, Bk, NULL, 0, fz, o2, lse2, keep2,
                                            margin2, slots2, om2, 1) == 0, "fwd_varlen_forced rc");
        free(fz); free(o2); free(lse2); free(om2); free(margin2); free(keep2); free(slots2);
    }
    double *dq = darr(nq, 0), *dk = darr(nk, 0), *dv = darr(nk, 0), *dqc = darr(nq, 0), *dkc = darr(nk, 0);
    rc = mala_oracle_bwd_varlen(q, k, v, o, dout, lse, cq, ck, B, Hq, Hkv, d, tau, Bq, Bk, NULL, 0, NULL, 0, dq, dk,
                                dv, keep, margin, dqc, dkc, 1);
    CHECK(rc == 0, "bwd_varlen rc");
    for (size_t i = 0; i < nk; ++i) CHECK(isfinite(dk[i]) && isfinite(dv[i]), "bwd_varlen dk, dv finite");
    free(cq); free(ck); free(q); free(k); free(v); free(dout); free(o); free(lse); free(margin); free(om); free(keep);
    free(slots); free(dq); free(dk); free(dv); free(dqc); free(dkc);
}

static void decode_case(int B, int N, int Hq, int Hkv, int d, double tau, int Bkd, int with_lens) {
    const int nT = (N + Bkd - 1) / Bkd;
    double *q = darr((size_t)B * Hq * d, 1), *kc = darr((size_t)B * N * Hkv * d, 1), *vc = darr((size_t)B * N * Hkv * d, 1);
    double *o = darr((size_t)B * Hq * d, 0), *lse = darr((size_t)B * Hq, 0), *margin = darr((size_t)B * Hkv * nT, 0);
    double* om = darr((size_t)B * Hq, 0);
    uint8_t* keep = (uint8_t*)calloc((size_t)B * Hkv * nT, 1);
    int32_t* kept = (int32_t*)calloc((size_t)B * Hkv, sizeof(int32_t));
    int32_t* lens = (int32_t*)malloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; ++b) lens[b] = 1 + (b * 7919) % N;
    int rc = mala_oracle_decode(q, kc, vc, B, N, Hq, Hkv, d, tau, Bkd, with_lens ? lens : NULL, o, lse, keep, margin,
                                kept, om, 1);
    CHECK(rc == 0, "decode rc");
    for (int i = 0; i < B * Hq; ++i) CHECK(isfinite(lse[i]), "decode lse finite");
    {
        uint8_t* fz = flip_every_third(keep, (size_t)B * Hkv * nT);
        if (with_lens)   /* tiles past a sequence's cache are not visited: keep has 0 there (calloc) */
            for (int b = 0; b < B; ++b)
                for (int kh = 0; kh < Hkv; ++kh)
                    for (int t = (lens[b] + Bkd - 1) / Bkd; t < nT; ++t) fz[((size_t)b * Hkv + kh) * nT + t] = 255;
        CHECK(mala_oracle_decode_forced(q, kc, vc, B, N, Hq, Hkv, d, tau, Bkd, with_lens ? lens : NULL, fz, o, lse,
                                        keep, margin, kept, om, 1) == 0, "decode_forced rc");
        free(fz);
    }
    lens[0] = N + 1;
    CHECK(mala_oracle_decode(q, kc, vc, B, N, Hq, Hkv, d, tau, Bkd, lens, o, lse, keep, margin, kept, om, 1) != 0,
          "decode refuses a cache length past N");
    free(q); free(kc); free(vc); free(o); free(lse); free(margin); free(om); free(keep); free(kept); free(lens);
}

int main(void) {
    const double taus[4] = {0.0, 0.25, 1.0, 4.0};
    for (int t = 0; t < 4; ++t) {
        fixed_case(1, 77, 4, 2, 8, taus[t], 32, 16, 0);
        fixed_case(2, 130, 3, 1, 16, taus[t], 64, 32, 0);
        fixed_case(1, 65, 2, 2, 4, taus[t], 1, 1, 0);
        fixed_case(1, 200, 6, 2, 8, taus[t], 128, 64, 1);
        fixed_case(1, 1, 2, 1, 8, taus[t], 64, 64, 0);
        const int lq[5] = {5, 0, 70, 1, 33}, lk[5] = {5, 13, 100, 64, 33};
        varlen_case(5, lq, lk, 4, 2, 8, taus[t], 32, 16);
        varlen_case(5, lq, lk, 2, 1, 8, taus[t], 1, 1);
        decode_case(3, 130, 6, 2, 8, taus[t], 64, 0);
        decode_case(4, 200, 5, 1, 16, taus[t], 16, 1);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitize driver: all calls OK\n");
    return 0;
}
