/*
 * wall_oracle.c -- plain fp64 CPU oracle for the Wall Attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP implementation and must never be
 * used as a fallback for it.
 *
 * What it computes (the plain definition, written out):
 *
 *   Wall Attention blog, section "Definition: Wall Attention", product form:
 *       o_i = sum_j softmax_j( sum_n F_{ij,n} q_{i,n} k_{j,n} ) v_j,
 *       F_{ij,n} = prod_{r=j+1..i} gate_{r,n}.
 *   wall-attention-release README ("Usage: Training / prefill"): the API
 *   argument g is the natural log of the gate (g = 0 is vanilla softmax
 *   attention), so gate_{r,n} = exp(g_{r,n}); `scale` multiplies the whole
 *   decayed dot product; HQ query heads share H key/value heads (HQ % H == 0).
 *   Optional arguments from the same README:
 *     g_scalar [B,T,HQ]  FoX-style additive gate: the logit of pair (i,j)
 *                        gains sum_{r=j+1..i} g_scalar_r (the blog's FoX
 *                        formula exp(q.k + log F_ij) in the section "Diagonal
 *                        forget gates in infinite dimensions"), unscaled;
 *     sink_bias [HQ]     one extra logit per query head with a zero value
 *                        vector; it takes part in the normalisation only;
 *     window_size W      key j is visible from query i iff 0 <= i-j < W;
 *     cu_seqlens         packed sequences (B == 1); no pair crosses a
 *                        sequence boundary.
 *   lse is the natural-log normaliser of each row, sink included, so that
 *   o_i = sum_j exp(logit_ij - lse_i) v_j.
 *
 * The loop below walks j from i down to the first visible key and keeps the
 * running product F (one factor exp(g_{j+1,n}) per step) and the running FoX
 * sum, so each logit is the literal product-form value.  Everything is fp64;
 * the softmax is the two-pass max / sum form.  OpenMP splits the (token,
 * head) rows; each row is computed independently and identically.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, a negative code on invalid arguments. */
int wall_oracle_fwd(const double *q,        /* [B,T,HQ,K] */
                    const double *k,        /* [B,T,H,K]  */
                    const double *v,        /* [B,T,H,V]  */
                    const double *g,        /* [B,T,HQ,K] natural-log gate */
                    const double *g_scalar, /* [B,T,HQ] or NULL */
                    const double *sink,     /* [HQ] or NULL */
                    double *o,              /* [B,T,HQ,V] */
                    double *lse,            /* [B,T,HQ] or NULL */
                    int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K,
                    int64_t V, double scale, int64_t window,
                    const int64_t *cu_seqlens, /* [nseq+1] or NULL (then B rows of T) */
                    int64_t nseq,
                    const int64_t *rows, /* flat token ids b*T+t to compute, or NULL = all */
                    int64_t nrows)
{
    if (!q || !k || !v || !g || !o) return -1;
    if (B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || V < 1) return -2;
    if (HQ % H != 0) return -3;
    if (cu_seqlens && (B != 1 || nseq < 1)) return -4;
    if (cu_seqlens) {
        if (cu_seqlens[0] != 0 || cu_seqlens[nseq] != T) return -5;
        for (int64_t s = 0; s < nseq; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return -5;
    }
    const int64_t group = HQ / H;
    const int64_t ntok = B * T;
    const int64_t nr = rows ? nrows : ntok;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= ntok) return -6;

    int fail = 0;
#pragma omp parallel
    {
        double *F = (double *)malloc(sizeof(double) * (size_t)K);
        double *logit = (double *)malloc(sizeof(double) * (size_t)T);
        double *acc = (double *)malloc(sizeof(double) * (size_t)V);
        if (!F || !logit || !acc) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1) collapse(2)
            for (int64_t r = 0; r < nr; ++r) {
                for (int64_t hq = 0; hq < HQ; ++hq) {
                    const int64_t tok = rows ? rows[r] : r;
                    const int64_t b = tok / T, i = tok % T;
                    /* start of the sequence that holds token i */
                    int64_t s0 = 0;
                    if (cu_seqlens) {
                        for (int64_t s = 0; s < nseq; ++s)
                            if (cu_seqlens[s] <= i && i < cu_seqlens[s + 1]) s0 = cu_seqlens[s];
                    }
                    int64_t lo = s0;
                    if (window > 0 && i - window + 1 > lo) lo = i - window + 1;
                    const int64_t h = hq / group;
                    const double *qi = q + ((b * T + i) * HQ + hq) * K;

                    for (int64_t n = 0; n < K; ++n) F[n] = 1.0;
                    double fox = 0.0;
                    int64_t cnt = 0;
                    for (int64_t j = i; j >= lo; --j) {
                        if (j < i) {
                            /* one more factor of the product over r = j+1 .. i */
                            const double *gr = g + ((b * T + (j + 1)) * HQ + hq) * K;
                            for (int64_t n = 0; n < K; ++n) F[n] *= exp(gr[n]);
                            if (g_scalar) fox += g_scalar[(b * T + (j + 1)) * HQ + hq];
                        }
                        const double *kj = k + ((b * T + j) * H + h) * K;
                        double dot = 0.0;
                        for (int64_t n = 0; n < K; ++n) dot += F[n] * qi[n] * kj[n];
                        logit[cnt++] = scale * dot + fox;
                    }
                    /* softmax over the visible keys (j = i, i-1, ..., lo) and the sink */
                    double m = -INFINITY;
                    for (int64_t c = 0; c < cnt; ++c) m = logit[c] > m ? logit[c] : m;
                    if (sink && sink[hq] > m) m = sink[hq];
                    double Z = 0.0;
                    for (int64_t d = 0; d < V; ++d) acc[d] = 0.0;
                    for (int64_t c = 0; c < cnt; ++c) {
                        const int64_t j = i - c;
                        const double p = exp(logit[c] - m);
                        Z += p;
                        const double *vj = v + ((b * T + j) * H + h) * V;
                        for (int64_t d = 0; d < V; ++d) acc[d] += p * vj[d];
                    }
                    if (sink) Z += exp(sink[hq] - m); /* value vector of the sink is zero */
                    double *oi = o + ((b * T + i) * HQ + hq) * V;
                    for (int64_t d = 0; d < V; ++d) oi[d] = acc[d] / Z;
                    if (lse) lse[(b * T + i) * HQ + hq] = m + log(Z);
                }
            }
        }
        free(F);
        free(logit);
        free(acc);
    }
    return fail ? -7 : 0;
}

/* Per-segment prefix sum along T, times `scale`:
 *   out[b,t,c] = scale * sum_{u = s(t) .. t} x[b,u,c]
 * where s(t) is the first token of the sequence holding t.  This is the
 * log-space prefix P_t = sum_{u<=t} log gate_u of the blog's factored form
 * ("Definition: Wall Attention"), expressed in log2 units when
 * scale = 1/ln 2 as the README's decode example does.  Rows are [C]
 * contiguous channels (C = HQ*K for g, HQ for g_scalar). */
int wall_oracle_prefix_scan(const double *x, double *out, int64_t B, int64_t T, int64_t C,
                            const int64_t *cu_seqlens, int64_t nseq, double scale)
{
    if (!x || !out || B < 1 || T < 1 || C < 1) return -1;
    if (cu_seqlens && (B != 1 || nseq < 1)) return -4;
#pragma omp parallel for collapse(2)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t c = 0; c < C; ++c) {
            double run = 0.0;
            int64_t s = 0;
            for (int64_t t = 0; t < T; ++t) {
                if (cu_seqlens) {
                    while (s < nseq && t >= cu_seqlens[s + 1]) ++s;
                    if (t == cu_seqlens[s]) run = 0.0;
                } else if (t == 0) {
                    run = 0.0;
                }
                run += x[(b * T + t) * C + c];
                out[(b * T + t) * C + c] = scale * run;
            }
        }
    }
    return 0;
}

/* Backward of the forward above (README: "exact analytic gradients" for q,
 * k, v, g and g_scalar), written from the product form.  With the logits
 * s_ij = scale * sum_n F_ij,n q_in k_jn + (Gs_i - Gs_j) (Gs the running sum
 * of g_scalar), A_ij = exp(s_ij - lse_i) and D_i = sum_v do_iv o_iv:
 *     dS_ij = A_ij (do_i . v_j - D_i)
 *     dv_j  = sum_i A_ij do_i                     (over the query heads of j's kv head)
 *     dq_in = scale sum_j dS_ij F_ij,n k_jn
 *     dk_jn = scale sum_i dS_ij F_ij,n q_in       (per query head, then summed)
 *     dsink = -sum_i exp(sink - lse_i) D_i
 * F_ij,n = prod_{r=j+1..i} exp(g_rn) depends on g_un for j < u <= i, so
 *     dg_un = sum_{i >= u > j} scale dS_ij F_ij,n q_in k_jn
 *           = sum_{t >= u, same sequence} (q_tn dq_tn - k_tn dk^(hq)_tn)
 * (the pairs with i >= u, minus those with j >= u, which also have i >= u),
 * and likewise dg_scalar_u = sum_{t >= u} (sum_j dS_tj - sum_i dS_it).
 * o and lse are recomputed here in fp64.  Outputs are overwritten; any of
 * dg_scalar / dsink may be NULL when g_scalar / sink is. */
int wall_oracle_bwd(const double *q, const double *k, const double *v, const double *g,
                    const double *g_scalar, const double *sink, const double *dout,
                    double *dq, double *dk, double *dv, double *dg, double *dgs, double *dsink,
                    int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                    double scale, int64_t window, const int64_t *cu_seqlens, int64_t nseq)
{
    if (!q || !k || !v || !g || !dout || !dq || !dk || !dv || !dg) return -1;
    if (B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || V < 1) return -2;
    if (HQ % H != 0) return -3;
    if (cu_seqlens && (B != 1 || nseq < 1)) return -4;
    const int64_t group = HQ / H;
    /* per query head: dk contributions and the two per-token sums whose
     * suffix sums give dg and dg_scalar */
    double *dkh = (double *)calloc((size_t)(B * T * HQ * K), sizeof(double));
    double *dvh = (double *)calloc((size_t)(B * T * HQ * V), sizeof(double));
    double *grow = (double *)calloc((size_t)(B * T * HQ), sizeof(double));
    double *gcol = (double *)calloc((size_t)(B * T * HQ), sizeof(double));
    double *sk = (double *)calloc((size_t)(B * HQ), sizeof(double));
    if (!dkh || !dvh || !grow || !gcol || !sk) {
        free(dkh); free(dvh); free(grow); free(gcol); free(sk);
        return -7;
    }
    int fail = 0;
#pragma omp parallel
    {
        double *F = (double *)malloc(sizeof(double) * (size_t)(K * T));
        double *logit = (double *)malloc(sizeof(double) * (size_t)T);
        double *o = (double *)malloc(sizeof(double) * (size_t)V);
        if (!F || !logit || !o) {
#pragma omp atomic write
            fail = 1;
        } else {
            /* one (b, hq) per task: its dk/dv/g sums are private to it */
#pragma omp for collapse(2) schedule(dynamic, 1)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t hq = 0; hq < HQ; ++hq) {
                    const int64_t hk = hq / group;
                    for (int64_t i = 0; i < T; ++i) {
                        int64_t s0 = 0;
                        if (cu_seqlens)
                            for (int64_t s = 0; s < nseq; ++s)
                                if (i >= cu_seqlens[s] && i < cu_seqlens[s + 1]) s0 = cu_seqlens[s];
                        int64_t lo = s0;
                        if (window > 0 && lo < i + 1 - window) lo = i + 1 - window;
                        const double *qi = q + ((b * T + i) * HQ + hq) * K;
                        const double *doi = dout + ((b * T + i) * HQ + hq) * V;
                        /* logits of row i, keeping F for every visible key (F[(i-j)*K + n]) */
                        double fox = 0.0;
                        for (int64_t j = i; j >= lo; --j) {
                            double *Fj = F + (i - j) * K;
                            if (j == i) {
                                for (int64_t n = 0; n < K; ++n) Fj[n] = 1.0;
                            } else {
                                const double *gj1 = g + ((b * T + j + 1) * HQ + hq) * K;
                                for (int64_t n = 0; n < K; ++n) Fj[n] = Fj[n - K] * exp(gj1[n]);
                                if (g_scalar) fox = fox + g_scalar[(b * T + j + 1) * HQ + hq];
                            }
                            const double *kj = k + ((b * T + j) * H + hk) * K;
                            double dot = 0.0;
                            for (int64_t n = 0; n < K; ++n) dot += Fj[n] * qi[n] * kj[n];
                            logit[i - j] = scale * dot + fox;
                        }
                        const int64_t cnt = i - lo + 1;
                        double m = -INFINITY;
                        for (int64_t c = 0; c < cnt; ++c) m = logit[c] > m ? logit[c] : m;
                        if (sink && sink[hq] > m) m = sink[hq];
                        double Z = 0.0;
                        for (int64_t c = 0; c < cnt; ++c) Z += exp(logit[c] - m);
                        if (sink) Z = Z + exp(sink[hq] - m);
                        const double lse = m + log(Z);
                        for (int64_t d = 0; d < V; ++d) o[d] = 0.0;
                        for (int64_t c = 0; c < cnt; ++c) {
                            const double *vj = v + ((b * T + (i - c)) * H + hk) * V;
                            const double a = exp(logit[c] - lse);
                            for (int64_t d = 0; d < V; ++d) o[d] += a * vj[d];
                        }
                        double Di = 0.0;
                        for (int64_t d = 0; d < V; ++d) Di += doi[d] * o[d];
                        if (sink) sk[b * HQ + hq] -= exp(sink[hq] - lse) * Di;
                        double *dqi = dq + ((b * T + i) * HQ + hq) * K;
                        for (int64_t n = 0; n < K; ++n) dqi[n] = 0.0;
                        for (int64_t c = 0; c < cnt; ++c) {
                            const int64_t j = i - c;
                            const double *vj = v + ((b * T + j) * H + hk) * V;
                            const double *kj = k + ((b * T + j) * H + hk) * K;
                            const double a = exp(logit[c] - lse);
                            double dpv = 0.0;
                            for (int64_t d = 0; d < V; ++d) dpv += doi[d] * vj[d];
                            const double dS = a * (dpv - Di);
                            const double *Fj = F + c * K;
                            double *dkj = dkh + ((b * T + j) * HQ + hq) * K;
                            double *dvj = dvh + ((b * T + j) * HQ + hq) * V;
                            for (int64_t n = 0; n < K; ++n) {
                                dqi[n] += scale * dS * Fj[n] * kj[n];
                                dkj[n] += scale * dS * Fj[n] * qi[n];
                            }
                            for (int64_t d = 0; d < V; ++d) dvj[d] += a * doi[d];
                            grow[(b * T + i) * HQ + hq] += dS;
                            gcol[(b * T + j) * HQ + hq] += dS;
                        }
                    }
                }
        }
        free(F);
        free(logit);
        free(o);
    }
    if (!fail) {
        /* dk, dv: sums over the query heads of each kv head */
        for (int64_t t = 0; t < B * T; ++t)
            for (int64_t h = 0; h < H; ++h) {
                double *dkt = dk + (t * H + h) * K;
                double *dvt = dv + (t * H + h) * V;
                for (int64_t n = 0; n < K; ++n) dkt[n] = 0.0;
                for (int64_t d = 0; d < V; ++d) dvt[d] = 0.0;
                for (int64_t hq = h * group; hq < (h + 1) * group; ++hq) {
                    for (int64_t n = 0; n < K; ++n) dkt[n] += dkh[(t * HQ + hq) * K + n];
                    for (int64_t d = 0; d < V; ++d) dvt[d] += dvh[(t * HQ + hq) * V + d];
                }
            }
        /* dg, dg_scalar: suffix sums within each sequence */
        for (int64_t b = 0; b < B; ++b)
            for (int64_t hq = 0; hq < HQ; ++hq) {
                const int64_t hk = hq / group;
                for (int64_t n = 0; n < K; ++n) {
                    double run = 0.0;
                    int64_t s = nseq - 1;
                    for (int64_t t = T - 1; t >= 0; --t) {
                        if (cu_seqlens) {
                            while (s > 0 && t < cu_seqlens[s]) --s;
                            if (t == cu_seqlens[s + 1] - 1) run = 0.0;
                        } else if (t == T - 1) {
                            run = 0.0;
                        }
                        const int64_t tk = (b * T + t) * HQ + hq;
                        run += q[tk * K + n] * dq[tk * K + n] - k[((b * T + t) * H + hk) * K + n] * dkh[tk * K + n];
                        dg[tk * K + n] = run;
                    }
                }
                if (dgs) {
                    double run = 0.0;
                    int64_t s = nseq - 1;
                    for (int64_t t = T - 1; t >= 0; --t) {
                        if (cu_seqlens) {
                            while (s > 0 && t < cu_seqlens[s]) --s;
                            if (t == cu_seqlens[s + 1] - 1) run = 0.0;
                        } else if (t == T - 1) {
                            run = 0.0;
                        }
                        const int64_t tk = (b * T + t) * HQ + hq;
                        run += grow[tk] - gcol[tk];
                        dgs[tk] = run;
                    }
                }
            }
        if (dsink)
            for (int64_t hq = 0; hq < HQ; ++hq) {
                double acc = 0.0;
                for (int64_t b = 0; b < B; ++b) acc += sk[b * HQ + hq];
                dsink[hq] = sink ? acc : 0.0;
            }
    }
    free(dkh);
    free(dvh);
    free(grow);
    free(gcol);
    free(sk);
    return fail ? -7 : 0;
}

/* Decode cache, wall-attention-release README ("Decode (cached generation)"):
 * the keys with the decay folded in, per chunk of C rows,
 *     k_tilde[b,j,hq,n] = k[b,j,h,n] * exp2(R[b,c,hq,n] - P[b,j,hq,n]),  c = j / C,
 * with one anchor R per chunk and channel.  The README names a per-chunk
 * anchor and its role, not its row; the reading taken here is the one an
 * append-as-you-go cache can keep while every cached factor stays in range:
 * R starts as the floor of P at the chunk's first row, and whenever a later
 * row t of the chunk has R - P[t] > CACHE_SPAN (its key factor would pass
 * 2^CACHE_SPAN) the anchor moves to floor(P[t]).  The rows before t are
 * then held against the new anchor too (k_tilde above always uses the final
 * R of the chunk).  CACHE_SPAN is 64 log2 units.
 * P is the log2 prefix [B,T,HQ,K] (prefix scan of g with scale 1/ln 2);
 * h = hq / (HQ/H).  r_cache is [B, ceil(T/C), HQ, K]. */
#define CACHE_SPAN 64.0
int wall_oracle_kv_cache(const double *k,  /* [B,T,H,K] */
                         const double *P,  /* [B,T,HQ,K] */
                         double *k_tilde,  /* [B,T,HQ,K] */
                         double *r_cache,  /* [B,NC,HQ,K] */
                         int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t C)
{
    if (!k || !P || !k_tilde || !r_cache) return -1;
    if (B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || C < 1) return -2;
    if (HQ % H != 0) return -3;
    const int64_t group = HQ / H, NC = (T + C - 1) / C;
#pragma omp parallel for collapse(3)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t c = 0; c < NC; ++c)
            for (int64_t hq = 0; hq < HQ; ++hq) {
                const int64_t kvh = hq / group;
                const int64_t j0 = c * C;
                const int64_t j1 = j0 + C < T ? j0 + C : T;
                double *R = r_cache + ((b * NC + c) * HQ + hq) * K;
                for (int64_t n = 0; n < K; ++n) {
                    double r = floor(P[((b * T + j0) * HQ + hq) * K + n]);
                    for (int64_t j = j0 + 1; j < j1; ++j) {
                        const double pj = P[((b * T + j) * HQ + hq) * K + n];
                        if (r - pj > CACHE_SPAN) r = floor(pj);
                    }
                    R[n] = r;
                }
                for (int64_t j = j0; j < j1; ++j) {
                    const double *kj = k + ((b * T + j) * H + kvh) * K;
                    const double *Pj = P + ((b * T + j) * HQ + hq) * K;
                    double *kt = k_tilde + ((b * T + j) * HQ + hq) * K;
                    for (int64_t n = 0; n < K; ++n) kt[n] = kj[n] * exp2(R[n] - Pj[n]);
                }
            }
    return 0;
}

/* Decode, wall-attention-release README (wall_attn_decode): one query per
 * (b, hq), at the row whose log2 prefix is p_curr, against every cached key
 * j = 0 .. T-1 of sequence b:
 *     logit_j = scale * sum_n q_n * exp2(p_curr_n - R[j / C, n]) * k_tilde[j, n],
 * which is the forward's logit scale * sum_n exp2(p_curr_n - P_j,n) q_n k_j,n
 * (the blog's factored form, "Definition: Wall Attention") with the anchor
 * cancelling.  The optional sink adds one logit with a zero value; lse is
 * the natural-log normaliser, sink included.  q, p_curr [B,HQ,K];
 * v [B,T,H,V]; o [B,HQ,V]; lse [B,HQ] or NULL. */
int wall_oracle_decode(const double *q, const double *v, const double *p_curr,
                       const double *k_tilde, const double *r_cache, const double *sink,
                       double *o, double *lse,
                       int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                       int64_t C, double scale)
{
    if (!q || !v || !p_curr || !k_tilde || !r_cache || !o) return -1;
    if (B < 1 || T < 1 || HQ < 1 || H < 1 || K < 1 || V < 1 || C < 1) return -2;
    if (HQ % H != 0) return -3;
    const int64_t group = HQ / H, NC = (T + C - 1) / C;
    int fail = 0;
#pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)T);
        double *acc = (double *)malloc(sizeof(double) * (size_t)V);
        if (!logit || !acc) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for collapse(2)
            for (int64_t b = 0; b < B; ++b)
                for (int64_t hq = 0; hq < HQ; ++hq) {
                    const int64_t kvh = hq / group;
                    const double *qi = q + (b * HQ + hq) * K;
                    const double *pc = p_curr + (b * HQ + hq) * K;
                    for (int64_t j = 0; j < T; ++j) {
                        const int64_t c = j / C;
                        const double *R = r_cache + ((b * NC + c) * HQ + hq) * K;
                        const double *kt = k_tilde + ((b * T + j) * HQ + hq) * K;
                        double dot = 0.0;
                        for (int64_t n = 0; n < K; ++n) dot += qi[n] * exp2(pc[n] - R[n]) * kt[n];
                        logit[j] = scale * dot;
                    }
                    double m = -INFINITY;
                    for (int64_t j = 0; j < T; ++j) m = logit[j] > m ? logit[j] : m;
                    if (sink && sink[hq] > m) m = sink[hq];
                    double Z = 0.0;
                    for (int64_t d = 0; d < V; ++d) acc[d] = 0.0;
                    for (int64_t j = 0; j < T; ++j) {
                        const double p = exp(logit[j] - m);
                        Z += p;
                        const double *vj = v + ((b * T + j) * H + kvh) * V;
                        for (int64_t d = 0; d < V; ++d) acc[d] += p * vj[d];
                    }
                    if (sink != NULL) Z += exp(sink[hq] - m);
                    double *oi = o + (b * HQ + hq) * V;
                    for (int64_t d = 0; d < V; ++d) oi[d] = acc[d] / Z;
                    if (lse) lse[b * HQ + hq] = m + log(Z);
                }
        }
        free(logit);
        free(acc);
    }
    return fail ? -7 : 0;
}

int wall_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
