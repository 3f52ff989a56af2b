/* Every function of oracle/wall_oracle.c on small seeded inputs, with
 * packed sequences, a window, a scalar gate, a sink, a row subset, and the
 * argument errors, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitize.py).  Checks return codes
 * and that every output written is finite; the values themselves are pinned
 * by the oracle's own tests.  Exits 0 on success, 1 otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int wall_oracle_fwd(const double *q, const double *k, const double *v, const double *g, const double *g_scalar,
                    const double *sink, double *o, double *lse, int64_t B, int64_t T, int64_t HQ, int64_t H,
                    int64_t K, int64_t V, double scale, int64_t window, const int64_t *cu_seqlens, int64_t nseq,
                    const int64_t *rows, int64_t nrows);
int wall_oracle_prefix_scan(const double *x, double *out, int64_t B, int64_t T, int64_t C,
                            const int64_t *cu_seqlens, int64_t nseq, double scale);
int wall_oracle_bwd(const double *q, const double *k, const double *v, const double *g, const double *g_scalar,
                    const double *sink, const double *dout, double *dq, double *dk, double *dv, double *dg,
                    double *dgs, double *dsink, int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                    double scale, int64_t window, const int64_t *cu_seqlens, int64_t nseq);
int wall_oracle_kv_cache(const double *k, const double *P, double *k_tilde, double *r_cache, int64_t B, int64_t T,
                         int64_t HQ, int64_t H, int64_t K, int64_t C);
int wall_oracle_decode(const double *q, const double *v, const double *p_curr, const double *k_tilde,
                       const double *r_cache, const double *sink, double *o, double *lse, int64_t B, int64_t T,
                       int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t C, double scale);
int wall_oracle_num_threads(void);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void) { /* xorshift64*, in [-1, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double *filled(size_t n, double lo, double hi) {
    double *p = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5 * (uniform() + 1.0);
    return p;
}
static int finite_all(const double *p, size_t n, const char *what) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) {
            fprintf(stderr, "%s[%zu] = %g\n", what, i, p[i]);
            return 0;
        }
    return 1;
}

int main(void) {
    enum { T = 70, HQ = 4, H = 2, K = 16, V = 8, C = 16 };
    const int64_t B = 1, nseq = 3, window = 20;
    const int64_t cu[4] = {0, 1, 33, T};
    const size_t nq = (size_t)B * T * HQ * K, nk = (size_t)B * T * H * K, nv = (size_t)B * T * H * V;
    double *q = filled(nq, -1, 1), *k = filled(nk, -1, 1), *v = filled(nv, -1, 1);
    double *g = filled(nq, -2.5, 0.0), *gs = filled((size_t)B * T * HQ, -0.1, 0.1), *sink = filled(HQ, -1, 1);
    double *dout = filled((size_t)B * T * HQ * V, -1, 1);
    double *o = (double *)calloc((size_t)B * T * HQ * V, sizeof(double)), *lse = (double *)calloc((size_t)B * T * HQ, sizeof(double));
    int ok = 1;

    /* forward: every row, then a subset of rows */
    ok &= wall_oracle_fwd(q, k, v, g, gs, sink, o, lse, B, T, HQ, H, K, V, 0.25, window, cu, nseq, NULL, 0) == 0;
    ok &= finite_all(o, (size_t)B * T * HQ * V, "o") && finite_all(lse, (size_t)B * T * HQ, "lse");
    const int64_t rows[3] = {0, 32, T - 1};
    ok &= wall_oracle_fwd(q, k, v, g, NULL, NULL, o, NULL, B, T, HQ, H, K, V, 0.25, 0, NULL, 0, rows, 3) == 0;
    ok &= wall_oracle_fwd(q, k, v, g, NULL, NULL, o, NULL, B, T, 3, H, K, V, 0.25, 0, NULL, 0, NULL, 0) != 0;
    const int64_t bad_row[1] = {T};
    ok &= wall_oracle_fwd(q, k, v, g, NULL, NULL, o, NULL, B, T, HQ, H, K, V, 0.25, 0, NULL, 0, bad_row, 1) != 0;

    /* prefix scan */
    double *P = (double *)malloc(nq * sizeof(double));
    ok &= wall_oracle_prefix_scan(g, P, B, T, HQ * K, cu, nseq, 1.0 / log(2.0)) == 0;
    ok &= finite_all(P, nq, "P");
    ok &= wall_oracle_prefix_scan(g, P, 2, T / 2, HQ * K, cu, nseq, 1.0) != 0;

    /* backward */
    double *dq = (double *)malloc(nq * sizeof(double)), *dk = (double *)malloc(nk * sizeof(double));
    double *dv = (double *)malloc(nv * sizeof(double)), *dg = (double *)malloc(nq * sizeof(double));
    double *dgs = (double *)malloc((size_t)B * T * HQ * sizeof(double)), *dsink = (double *)malloc(HQ * sizeof(double));
    ok &= wall_oracle_bwd(q, k, v, g, gs, sink, dout, dq, dk, dv, dg, dgs, dsink, B, T, HQ, H, K, V, 0.25, window,
                          cu, nseq) == 0;
    ok &= finite_all(dq, nq, "dq") && finite_all(dk, nk, "dk") && finite_all(dv, nv, "dv") &&
          finite_all(dg, nq, "dg") && finite_all(dgs, (size_t)B * T * HQ, "dgs") && finite_all(dsink, HQ, "dsink");
    ok &= wall_oracle_bwd(q, k, v, g, NULL, NULL, dout, NULL, dk, dv, dg, NULL, NULL, B, T, HQ, H, K, V, 0.25, 0,
                          NULL, 0) != 0;

    /* decode cache and decode (two sequences of T rows: reuse the first B*T rows twice) */
    const int64_t NC = (T + C - 1) / C;
    double *kt = (double *)malloc(nq * sizeof(double)), *r = (double *)malloc((size_t)NC * HQ * K * sizeof(double));
    ok &= wall_oracle_kv_cache(k, P, kt, r, B, T, HQ, H, K, C) == 0;
    ok &= finite_all(kt, nq, "k_tilde") && finite_all(r, (size_t)NC * HQ * K, "r_cache");
    ok &= wall_oracle_kv_cache(k, P, kt, r, B, T, HQ, H, K, 0) != 0;
    double *od = (double *)malloc((size_t)HQ * V * sizeof(double)), *ld = (double *)malloc(HQ * sizeof(double));
    const double *pcur = P + (size_t)(T - 1) * HQ * K;
    const double *qlast = q + (size_t)(T - 1) * HQ * K;
    ok &= wall_oracle_decode(qlast, v, pcur, kt, r, sink, od, ld, B, T, HQ, H, K, V, C, 0.25) == 0;
    ok &= finite_all(od, (size_t)HQ * V, "decode o") && finite_all(ld, HQ, "decode lse");
    ok &= wall_oracle_decode(qlast, v, pcur, kt, r, sink, od, ld, B, T, HQ, 3, K, V, C, 0.25) != 0;
    ok &= wall_oracle_num_threads() >= 1;

    free(q); free(k); free(v); free(g); free(gs); free(sink); free(dout); free(o); free(lse); free(P);
    free(dq); free(dk); free(dv); free(dg); free(dgs); free(dsink); free(kt); free(r); free(od); free(ld);
    if (!ok) {
        fprintf(stderr, "oracle checks failed\n");
        return 1;
    }
    printf("oracle checks passed\n");
    return 0;
}
