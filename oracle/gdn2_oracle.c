/*
 * gdn2_oracle.c -- plain, slow, float64 CPU oracle of the Gated DeltaNet-2
 * (GDN-2) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU library; the product path never calls it.
 *
 * What it computes (one head, state S in R^{dk x dv}, key channel = row i,
 * value channel = column j), token by token, in the order the pages give:
 *
 *   1. decay first: D = Diag(alpha_t) S_{t-1}, a per-key-channel decay
 *      inherited from KDA ("Gated DeltaNet-2", aixai.ru blog, section "One
 *      scalar cannot decide two different questions", formal paragraph; the
 *      gate tables on needhelp.icu/fa and needhelp.icu/de).
 *   2. read with the erase-gated key: r = D^T (b_t (.) k_t); in this reading
 *      b enters the read of the state (same paragraph).
 *   3. delta value with the write-gated candidate: z = w_t (.) v_t - r; the
 *      write gate sits on the value side (aiexpert.news/pt, method paragraph:
 *      b_t in [0,1]^dk on the key axis, w_t in [0,1]^dv on the value axis).
 *   4. one rank-1 write along the key: S_t = D + k_t z^T.
 *   5. read-out after the update: o_t = S_t^T q_t (no 1/sqrt(dk) scale).
 *
 * With b_t = w_t = beta_t * 1 this is KDA exactly; with a scalar decay as well
 * it is Gated DeltaNet; with alpha = 1 it is DeltaNet (aiexpert.news/pt,
 * method paragraph; needhelp.icu/de, section "Generalisierungshierarchie").
 *
 * Rule 1 (ORACLE_RULE_R1) is the alternative reading in which b only places
 * the erase and the read uses the plain key:
 *   r = D^T k_t;  S_t = D - (b_t (.) k_t) r^T + k_t (w_t (.) v_t)^T.
 * It is kept for comparison; the GPU path implements rule 0.
 *
 * Layout: inputs [B, T, H, d] token-major; state [N, H, dk, dv]; with
 * cu_seqlens (length N+1, B must be 1) sequence n covers tokens
 * cu_seqlens[n] .. cu_seqlens[n+1]-1; without it, sequence n is batch row n.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_RULE_R5 0
#define ORACLE_RULE_R1 1

/* One token of the recurrence on one head.  S is dk x dv row-major and is
 * updated in place; o receives dv values.  Scratch r, z have dv entries. */
static void gdn2_token_step(double *S, int dk, int dv,
                            const double *q, const double *k, const double *v,
                            const double *alpha, const double *b, const double *w,
                            int rule, double *r, double *z, double *o)
{
    int i, j;
    /* 1. decay each key-channel row of S */
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] *= alpha[i];
    /* 2. read */
    for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i) {
            double key = (rule == ORACLE_RULE_R5) ? b[i] * k[i] : k[i];
            acc += key * S[(size_t)i * dv + j];
        }
        r[j] = acc;
    }
    if (rule == ORACLE_RULE_R5) {
        /* 3. delta value, 4. rank-1 write along k */
        for (j = 0; j < dv; ++j)
            z[j] = w[j] * v[j] - r[j];
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] += k[i] * z[j];
    } else {
        /* R1: erase along the gated key, write along the plain key */
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] += -b[i] * k[i] * r[j] + k[i] * w[j] * v[j];
    }
    /* 5. read-out after the update */
    for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i)
            acc += q[i] * S[(size_t)i * dv + j];
        o[j] = acc;
    }
}

int gdn2_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void gdn2_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Full forward.  Returns 0 on success, -1 on bad arguments, -2 on allocation
 * failure.  S0 may be NULL (zero initial state); S_final may be NULL. */
int gdn2_oracle_fwd(const double *q, const double *k, const double *v,
                    const double *alpha, const double *b, const double *w,
                    const double *S0, const int32_t *cu_seqlens,
                    int B, int T, int H, int dk, int dv, int num_seqs, int rule,
                    double *o, double *S_final)
{
    int n_units;
    int bad = 0;
    if (!q || !k || !v || !alpha || !b || !w || !o)
        return -1;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (cu_seqlens) {
        int n;
        if (B != 1 || num_seqs <= 0 || cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T)
            return -1;
        for (n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n])
                return -1;
    } else {
        num_seqs = B;
    }
    n_units = num_seqs * H;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int u = 0; u < n_units; ++u) {
        int n = u / H, h = u % H;
        long t0, t1, t;
        size_t bt;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        double *z = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !r || !z) {
            free(S); free(r); free(z);
            bad |= 1;
            continue;
        }
        if (S0)
            memcpy(S, S0 + ((size_t)n * H + h) * dk * dv, sizeof(double) * (size_t)dk * dv);
        else
            memset(S, 0, sizeof(double) * (size_t)dk * dv);
        if (cu_seqlens) {
            t0 = cu_seqlens[n];
            t1 = cu_seqlens[n + 1];
            bt = 0;
        } else {
            t0 = 0;
            t1 = T;
            bt = (size_t)n * T;
        }
        for (t = t0; t < t1; ++t) {
            size_t row = (bt + (size_t)t) * H + h;
            gdn2_token_step(S, dk, dv, q + row * dk, k + row * dk, v + row * dv,
                            alpha + row * dk, b + row * dk, w + row * dv, rule, r, z,
                            o + row * dv);
        }
        if (S_final)
            memcpy(S_final + ((size_t)n * H + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S); free(r); free(z);
    }
    return bad ? -2 : 0;
}

/* One decode step for N sequences x H heads: inputs [N, H, d], state
 * [N, H, dk, dv] updated in place, o [N, H, dv]. */
int gdn2_oracle_decode(const double *q, const double *k, const double *v,
                       const double *alpha, const double *b, const double *w,
                       double *S, int N, int H, int dk, int dv, int rule, double *o)
{
    int bad = 0;
    if (!q || !k || !v || !alpha || !b || !w || !S || !o)
        return -1;
    if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int u = 0; u < N * H; ++u) {
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        double *z = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!r || !z) {
            free(r); free(z);
            bad |= 1;
            continue;
        }
        gdn2_token_step(S + (size_t)u * dk * dv, dk, dv, q + (size_t)u * dk, k + (size_t)u * dk,
                        v + (size_t)u * dv, alpha + (size_t)u * dk, b + (size_t)u * dk,
                        w + (size_t)u * dv, rule, r, z, o + (size_t)u * dv);
        free(r); free(z);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------ backward
 * Gradients of a scalar loss L through the rule-0 forward above, given
 * dL/do (do_) for every token and dL/dS_final (dSf, NULL = zero).  This is
 * the reverse-mode derivative of the five token steps, taken one token at a
 * time from the last to the first ("Gated DeltaNet-2", aixai.ru blog, formal
 * paragraph, differentiated by hand; the pages require gradients through both
 * gates, aiexpert.news/pt, method paragraph).  With dS = dL/dS_t carried
 * backwards, for token t (S_prev = S_{t-1}, D = Diag(alpha) S_prev,
 * e = b (.) k, z = w (.) v - D^T e, S_t = D + k z^T, o = S_t^T q):
 *   dS  += q do^T            dq = S_t do
 *   dk   = dS z              dz = dS^T k
 *   dw   = dz (.) v          dv = dz (.) w
 *   dD   = dS - e dz^T       de = -D dz
 *   db   = de (.) k          dk += de (.) b
 *   dalpha_i = sum_j dD_ij S_prev_ij
 *   dS_{t-1} = Diag(alpha) dD
 * The states are recomputed from checkpoints every SEG tokens (the same
 * arithmetic as the forward, so the same values), which bounds memory.
 */
#define ORACLE_BWD_SEG 64

static void gdn2_token_bwd(const double *Sp, const double *St, double *dS, int dk, int dv,
                           const double *q, const double *k, const double *v,
                           const double *alpha, const double *b, const double *w,
                           const double *dout, double *z, double *dz, double *de,
                           double *dq, double *dkk, double *dvv, double *dal, double *db,
                           double *dw)
{
    int i, j;
    /* recompute z from S_prev */
    for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i)
            acc += b[i] * k[i] * alpha[i] * Sp[(size_t)i * dv + j];
        z[j] = w[j] * v[j] - acc;
    }
    /* output read: o = S_t^T q */
    for (i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (j = 0; j < dv; ++j) {
            dS[(size_t)i * dv + j] += q[i] * dout[j];
            acc += St[(size_t)i * dv + j] * dout[j];
        }
        dq[i] = acc;
    }
    /* rank-1 write S_t = D + k z^T */
    for (i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (j = 0; j < dv; ++j)
            acc += dS[(size_t)i * dv + j] * z[j];
        dkk[i] = acc;
    }
    for (j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (i = 0; i < dk; ++i)
            acc += dS[(size_t)i * dv + j] * k[i];
        dz[j] = acc;
        dw[j] = acc * v[j];
        dvv[j] = acc * w[j];
    }
    /* read r = D^T e enters z with a minus sign: de = -D dz */
    for (i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (j = 0; j < dv; ++j)
            acc += alpha[i] * Sp[(size_t)i * dv + j] * dz[j];
        de[i] = -acc;
        db[i] = de[i] * k[i];
        dkk[i] += de[i] * b[i];
    }
    /* dD = dS - e dz^T; decay D = Diag(alpha) S_prev */
    for (i = 0; i < dk; ++i) {
        double e = b[i] * k[i], acc = 0.0;
        for (j = 0; j < dv; ++j) {
            double dD = dS[(size_t)i * dv + j] - e * dz[j];
            acc += dD * Sp[(size_t)i * dv + j];
            dS[(size_t)i * dv + j] = alpha[i] * dD;
        }
        dal[i] = acc;
    }
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 * S0, dSf and dS0 may be NULL.  Every gradient has its input's layout. */
int gdn2_oracle_bwd(const double *q, const double *k, const double *v,
                    const double *alpha, const double *b, const double *w,
                    const double *S0, const int32_t *cu_seqlens,
                    int B, int T, int H, int dk, int dv, int num_seqs,
                    const double *dout, const double *dSf,
                    double *dq, double *dk_out, double *dv_out, double *dalpha,
                    double *db, double *dw, double *dS0)
{
    int n_units;
    int bad = 0;
    if (!q || !k || !v || !alpha || !b || !w || !dout)
        return -1;
    if (!dq || !dk_out || !dv_out || !dalpha || !db || !dw)
        return -1;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (cu_seqlens) {
        int n;
        if (B != 1 || num_seqs <= 0 || cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T)
            return -1;
        for (n = 0; n < num_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n])
                return -1;
    } else {
        num_seqs = B;
    }
    n_units = num_seqs * H;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int u = 0; u < n_units; ++u) {
        int n = u / H, h = u % H;
        long t0, t1, len, nseg, sg, t;
        size_t bt, SS = (size_t)dk * dv;
        double *ck, *seg, *dS, *r, *z, *dz, *de, *otmp;
        if (cu_seqlens) {
            t0 = cu_seqlens[n];
            t1 = cu_seqlens[n + 1];
            bt = 0;
        } else {
            t0 = 0;
            t1 = T;
            bt = (size_t)n * T;
        }
        len = t1 - t0;
        nseg = (len + ORACLE_BWD_SEG - 1) / ORACLE_BWD_SEG;
        ck = (double *)malloc(sizeof(double) * SS * (size_t)(nseg > 0 ? nseg : 1));
        seg = (double *)malloc(sizeof(double) * SS * (ORACLE_BWD_SEG + 1));
        dS = (double *)malloc(sizeof(double) * SS);
        r = (double *)malloc(sizeof(double) * (size_t)dv);
        z = (double *)malloc(sizeof(double) * (size_t)dv);
        dz = (double *)malloc(sizeof(double) * (size_t)dv);
        otmp = (double *)malloc(sizeof(double) * (size_t)dv);
        de = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!ck || !seg || !dS || !r || !z || !dz || !otmp || !de) {
            free(ck); free(seg); free(dS); free(r); free(z); free(dz); free(otmp); free(de);
            bad |= 1;
            continue;
        }
        /* forward pass keeping the state entering every segment */
        if (S0)
            memcpy(seg, S0 + ((size_t)n * H + h) * SS, sizeof(double) * SS);
        else
            memset(seg, 0, sizeof(double) * SS);
        for (sg = 0; sg < nseg; ++sg) {
            long ta = t0 + sg * ORACLE_BWD_SEG;
            long tb = ta + ORACLE_BWD_SEG < t1 ? ta + ORACLE_BWD_SEG : t1;
            memcpy(ck + (size_t)sg * SS, seg, sizeof(double) * SS);
            for (t = ta; t < tb; ++t) {
                size_t row = (bt + (size_t)t) * H + h;
                gdn2_token_step(seg, dk, dv, q + row * dk, k + row * dk, v + row * dv,
                                alpha + row * dk, b + row * dk, w + row * dv, ORACLE_RULE_R5,
                                r, z, otmp);
            }
        }
        /* backward, segment by segment from the last */
        if (dSf)
            memcpy(dS, dSf + ((size_t)n * H + h) * SS, sizeof(double) * SS);
        else
            memset(dS, 0, sizeof(double) * SS);
        for (sg = nseg - 1; sg >= 0; --sg) {
            long ta = t0 + sg * ORACLE_BWD_SEG;
            long tb = ta + ORACLE_BWD_SEG < t1 ? ta + ORACLE_BWD_SEG : t1;
            memcpy(seg, ck + (size_t)sg * SS, sizeof(double) * SS);
            for (t = ta; t < tb; ++t) {
                size_t row = (bt + (size_t)t) * H + h;
                double *Sn = seg + (size_t)(t - ta + 1) * SS;
                memcpy(Sn, Sn - SS, sizeof(double) * SS);
                gdn2_token_step(Sn, dk, dv, q + row * dk, k + row * dk, v + row * dv,
                                alpha + row * dk, b + row * dk, w + row * dv, ORACLE_RULE_R5,
                                r, z, otmp);
            }
            for (t = tb - 1; t >= ta; --t) {
                size_t row = (bt + (size_t)t) * H + h;
                const double *Sp = seg + (size_t)(t - ta) * SS;
                gdn2_token_bwd(Sp, Sp + SS, dS, dk, dv, q + row * dk, k + row * dk,
                               v + row * dv, alpha + row * dk, b + row * dk, w + row * dv,
                               dout + row * dv, z, dz, de, dq + row * dk, dk_out + row * dk,
                               dv_out + row * dv, dalpha + row * dk, db + row * dk,
                               dw + row * dv);
            }
        }
        if (dS0)
            memcpy(dS0 + ((size_t)n * H + h) * SS, dS, sizeof(double) * SS);
        free(ck); free(seg); free(dS); free(r); free(z); free(dz); free(otmp); free(de);
    }
    return bad ? -2 : 0;
}
