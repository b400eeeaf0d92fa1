/*
 * kda_oracle.c -- plain, slow fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) per-head recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path
 * (libkda) never calls it, links it or shares code with it.
 *
 * Source of the method: page "Kimi K3 把 3T 级模型、百万上下文和 Agent 训练接成
 * 一套系统" (ailearn.mscapital.top/kimi-k3.html), card "KDA 单头递归":
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *
 * alpha says how much each channel forgets, beta how strongly the token
 * writes, the old state is decayed per channel first and then corrected and
 * written with the delta rule, and the query reads the *updated* state.
 * Readings taken where the page is silent (each is listed in the design doc):
 *   - alpha_t = exp(g_t), natural exponential, g_t given per channel;
 *   - S is dk x dv (row index = key channel, column = value channel) and the
 *     output is o_t = S_t^T q_t;
 *   - no scaling, normalisation, gating or convolution happens inside the
 *     recurrence; a NULL initial state means zeros;
 *   - an empty sequence produces no outputs and final = initial state.
 *
 * Expanding the page's product, with Sbar = Diag(alpha_t) S_{t-1}:
 *     S_t = Sbar - beta_t k_t (k_t^T Sbar) + beta_t k_t v_t^T
 *         = Sbar + beta_t k_t u_t^T,   u_t = v_t - Sbar^T k_t,
 * which is the token step below (decay, read-back, rank-1 write, read-out).
 * The test suite pins this against the page's product form written out with
 * explicit dk x dk matrices, a hand-worked example and closed forms.
 *
 * All arithmetic is fp64 (inputs are fp32 arrays holding the exact values the
 * device path sees, e.g. bf16 values widened to fp32).  No blocking, no
 * reordering beyond the definition; OpenMP only distributes independent
 * (sequence, head) units over threads, longest sequence first.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on one (sequence, head) state.
 * S: dk x dv row-major fp64, updated in place.  u, o: dv fp64 scratch/out. */
static void kda_token_step(double *S, int dk, int dv,
                           const float *q, const float *k, const float *v,
                           const float *g, double beta, double *u, double *o)
{
    /* decay first: row c of S is multiplied by alpha_c = exp(g_c) */
    for (int c = 0; c < dk; ++c) {
        const double a = exp((double)g[c]);
        double *row = S + (size_t)c * dv;
        for (int j = 0; j < dv; ++j) row[j] *= a;
    }
    /* delta-rule correction target: u = v - Sbar^T k */
    for (int j = 0; j < dv; ++j) u[j] = (double)v[j];
    for (int c = 0; c < dk; ++c) {
        const double kc = (double)k[c];
        const double *row = S + (size_t)c * dv;
        for (int j = 0; j < dv; ++j) u[j] -= row[j] * kc;
    }
    /* write: S = Sbar + beta k u^T */
    for (int c = 0; c < dk; ++c) {
        const double bk = beta * (double)k[c];
        double *row = S + (size_t)c * dv;
        for (int j = 0; j < dv; ++j) row[j] += bk * u[j];
    }
    /* the query reads the updated state: o = S_t^T q */
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
        const double qc = (double)q[c];
        const double *row = S + (size_t)c * dv;
        for (int j = 0; j < dv; ++j) o[j] += row[j] * qc;
    }
}

typedef struct { int32_t n, h, len; } unit_t;

static int cmp_len_desc(const void *a, const void *b)
{
    const unit_t *x = (const unit_t *)a, *y = (const unit_t *)b;
    if (x->len != y->len) return (y->len > x->len) ? 1 : -1;
    if (x->n != y->n) return x->n - y->n;
    return x->h - y->h;
}

/*
 * Prefill over packed variable-length sequences.
 *   q, k: [T_tot, H, dk] fp32;  v: [T_tot, H, dv] fp32;  g: [T_tot, H, dk] fp32
 *   beta: [T_tot, H] fp32
 *   initial_state: [N, H, dk, dv] fp64 or NULL (zeros)
 *   cu_seqlens: host [N+1], cu[0] = 0, non-decreasing, cu[N] = T_tot
 *   out: [T_tot, H, dv] fp64 (fully written for tokens inside [0, cu[N]))
 *   final_state: [N, H, dk, dv] fp64 or NULL
 *   num_threads <= 0 means the OpenMP default.
 * Returns 0 on success, 1 on invalid arguments, 2 on allocation failure.
 */
int kda_oracle_prefill(const float *q, const float *k, const float *v,
                       const float *g, const float *beta,
                       const double *initial_state, const int32_t *cu_seqlens,
                       int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv,
                       double *out, double *final_state, int32_t num_threads)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !out) return 1;
    if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0) return 1;
    if (cu_seqlens[0] != 0) return 1;
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;

    const int64_t nunits = (int64_t)num_seqs * num_heads;
    unit_t *units = (unit_t *)malloc(sizeof(unit_t) * (size_t)(nunits ? nunits : 1));
    if (!units) return 2;
    for (int32_t n = 0; n < num_seqs; ++n)
        for (int32_t h = 0; h < num_heads; ++h) {
            unit_t *u = &units[(int64_t)n * num_heads + h];
            u->n = n; u->h = h; u->len = cu_seqlens[n + 1] - cu_seqlens[n];
        }
    qsort(units, (size_t)nunits, sizeof(unit_t), cmp_len_desc);

    int failed = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !u) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nunits; ++i) {
            if (!S || !u) continue;
            const int32_t n = units[i].n, h = units[i].h;
            const size_t sidx = ((size_t)n * num_heads + h) * (size_t)dk * dv;
            if (initial_state)
                memcpy(S, initial_state + sidx, sizeof(double) * (size_t)dk * dv);
            else
                memset(S, 0, sizeof(double) * (size_t)dk * dv);
            for (int32_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
                const size_t th = (size_t)t * num_heads + h;
                kda_token_step(S, dk, dv, q + th * dk, k + th * dk, v + th * dv,
                               g + th * dk, (double)beta[th], u, out + th * dv);
            }
            if (final_state)
                memcpy(final_state + sidx, S, sizeof(double) * (size_t)dk * dv);
        }
        free(S);
        free(u);
    }
    free(units);
    return failed ? 2 : 0;
}

/*
 * One decode step: the same token step applied to one new token per
 * (sequence, head), with the state read-modified-written in place.
 *   q, k: [N, H, dk]; v: [N, H, dv]; g: [N, H, dk]; beta: [N, H]   (fp32)
 *   state_inout: [N, H, dk, dv] fp64;  out: [N, H, dv] fp64
 */
int kda_oracle_decode_step(const float *q, const float *k, const float *v,
                           const float *g, const float *beta, double *state_inout,
                           int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv,
                           double *out, int32_t num_threads)
{
    if (!q || !k || !v || !g || !beta || !state_inout || !out) return 1;
    if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0) return 1;
    const int64_t nunits = (int64_t)num_seqs * num_heads;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
#pragma omp parallel
    {
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!u) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nunits; ++i) {
            if (!u) continue;
            kda_token_step(state_inout + (size_t)i * dk * dv, dk, dv,
                           q + (size_t)i * dk, k + (size_t)i * dk, v + (size_t)i * dv,
                           g + (size_t)i * dk, (double)beta[i], u, out + (size_t)i * dv);
        }
        free(u);
    }
    return failed ? 2 : 0;
}

/*
 * Backward pass (gradients of a scalar loss through the recurrence), by the
 * chain rule applied to the token step in reverse order.  With Sp = S_{t-1},
 * Sbar = Diag(alpha) Sp, u = v - Sbar^T k, S = Sbar + beta k u^T, o = S^T q,
 * and dS the loss gradient with respect to S_t (from later tokens and, at the
 * end, d(final_state)):
 *     dS   += q do^T;                      dq = S do
 *     du    = beta dS^T k;                 dbeta = k^T dS u;   dk = beta dS u
 *     dv    = du;   dSbar = dS - k du^T;   dk -= Sbar du
 *     dalpha = rowsum(dSbar (.) Sp);       dg = alpha (.) dalpha
 *     dS_{t-1} = Diag(alpha) dSbar
 * and d(initial_state) = dS after the first token.  Each unit keeps all its
 * states S_0 .. S_T (fp64), so this is meant for test-sized inputs.
 *   dout: [T_tot, H, dv] fp64;  dfinal: [N, H, dk, dv] fp64 or NULL (zero)
 *   dq, dk, dg: [T_tot, H, dk] fp64;  dv: [T_tot, H, dv] fp64;
 *   dbeta: [T_tot, H] fp64;  dinit: [N, H, dk, dv] fp64 or NULL
 * Returns 0 on success, 1 on invalid arguments, 2 on allocation failure.
 */
int kda_oracle_backward(const float *q, const float *k, const float *v,
                        const float *g, const float *beta,
                        const double *initial_state, const int32_t *cu_seqlens,
                        int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv,
                        const double *dout, const double *dfinal,
                        double *dq, double *dk_out, double *dv_out, double *dg, double *dbeta,
                        double *dinit, int32_t num_threads)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !dout) return 1;
    if (!dq || !dk_out || !dv_out || !dg || !dbeta) return 1;
    if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0) return 1;
    if (cu_seqlens[0] != 0) return 1;
    for (int32_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 1;
    const int64_t nunits = (int64_t)num_seqs * num_heads;
    const size_t SS = (size_t)dk * dv;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nunits; ++i) {
        const int32_t n = (int32_t)(i / num_heads), h = (int32_t)(i % num_heads);
        const int32_t t0 = cu_seqlens[n], len = cu_seqlens[n + 1] - cu_seqlens[n];
        const size_t sidx = ((size_t)n * num_heads + h) * SS;
        double *S = (double *)malloc(sizeof(double) * SS * ((size_t)len + 1));
        double *dS = (double *)malloc(sizeof(double) * SS);
        double *Sbar = (double *)malloc(sizeof(double) * SS);
        double *u = (double *)malloc(sizeof(double) * dv);
        double *o = (double *)malloc(sizeof(double) * dv);
        double *du = (double *)malloc(sizeof(double) * dv);
        if (!S || !dS || !Sbar || !u || !o || !du) {
#pragma omp atomic write
            failed = 1;
        } else {
            /* forward, keeping every state */
            if (initial_state) memcpy(S, initial_state + sidx, sizeof(double) * SS);
            else memset(S, 0, sizeof(double) * SS);
            for (int32_t t = 0; t < len; ++t) {
                const size_t th = (size_t)(t0 + t) * num_heads + h;
                memcpy(S + (size_t)(t + 1) * SS, S + (size_t)t * SS, sizeof(double) * SS);
                kda_token_step(S + (size_t)(t + 1) * SS, dk, dv, q + th * dk, k + th * dk, v + th * dv,
                               g + th * dk, (double)beta[th], u, o);
            }
            /* reverse */
            if (dfinal) memcpy(dS, dfinal + sidx, sizeof(double) * SS);
            else memset(dS, 0, sizeof(double) * SS);
            for (int32_t t = len - 1; t >= 0; --t) {
                const size_t th = (size_t)(t0 + t) * num_heads + h;
                const float *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv, *gt = g + th * dk;
                const double bt = (double)beta[th];
                const double *Sp = S + (size_t)t * SS, *Sn = S + (size_t)(t + 1) * SS;
                const double *dot = dout + th * dv;
                /* recompute Sbar and u of this token */
                for (int c = 0; c < dk; ++c) {
                    const double a = exp((double)gt[c]);
                    for (int j = 0; j < dv; ++j) Sbar[(size_t)c * dv + j] = a * Sp[(size_t)c * dv + j];
                }
                for (int j = 0; j < dv; ++j) {
                    double s = (double)vt[j];
                    for (int c = 0; c < dk; ++c) s -= Sbar[(size_t)c * dv + j] * (double)kt[c];
                    u[j] = s;
                }
                /* o = S^T q */
                for (int c = 0; c < dk; ++c) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        dS[(size_t)c * dv + j] += (double)qt[c] * dot[j];
                        s += Sn[(size_t)c * dv + j] * dot[j];
                    }
                    dq[th * dk + c] = s;
                }
                /* S = Sbar + beta k u^T */
                double db = 0.0;
                for (int j = 0; j < dv; ++j) {
                    double s = 0.0;
                    for (int c = 0; c < dk; ++c) s += dS[(size_t)c * dv + j] * (double)kt[c];
                    du[j] = bt * s;
                    db += s * u[j];
                }
                dbeta[th] = db;
                for (int c = 0; c < dk; ++c) {
                    double s = 0.0, r = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        s += dS[(size_t)c * dv + j] * u[j];
                        r += Sbar[(size_t)c * dv + j] * du[j];
                    }
                    dk_out[th * dk + c] = bt * s - r;   /* write term, then u = v - Sbar^T k */
                }
                for (int j = 0; j < dv; ++j) dv_out[th * dv + j] = du[j];
                /* dSbar = dS - k du^T, then Sbar = Diag(alpha) Sp */
                for (int c = 0; c < dk; ++c) {
                    const double a = exp((double)gt[c]);
                    double da = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        const double dsb = dS[(size_t)c * dv + j] - (double)kt[c] * du[j];
                        da += dsb * Sp[(size_t)c * dv + j];
                        dS[(size_t)c * dv + j] = a * dsb;
                    }
                    dg[th * dk + c] = a * da;
                }
            }
            if (dinit) memcpy(dinit + sidx, dS, sizeof(double) * SS);
        }
        free(S); free(dS); free(Sbar); free(u); free(o); free(du);
    }
    return failed ? 2 : 0;
}
