/*
 * gdn2_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU evaluation of the Gated DeltaNet-2 recurrence (and of its
 * gradient, gdn2_oracle_sequence_bwd, at the end of the file). It exists
 * to check the GPU library; only the test suite, the smoke entry point and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header or helper
 * with the GPU library.
 *
 * What it computes (burn-gdn2 0.1.5 docs page, section "Architecture", the per-token
 * recurrence on the matrix state S in R^{d_k x d_v}):
 *
 *     S_t = (I - k_t (b_t (.) k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t (.) v_t)^T
 *     o_t = q_t^T S_t
 *
 * b_t is the erase gate on the key axis, w_t the write gate on the value axis, and
 * alpha_t the channel-wise decay on the key axis. Readings taken where the page is
 * silent:
 *   - o_t reads the state after the update of token t (the equation names S with
 *     no index; the GDN decode verify page, section 2, reads out after the rank-1
 *     update).
 *   - the decay is passed as log(alpha_t) <= 0 and exponentiated here (the llama.cpp
 *     notes, section 2, carry the decay as g and apply exp(g)).
 *   - no query scaling is applied.
 *
 * The erase matrix (I - k (b.k)^T) is applied to the decayed state without forming
 * it: (I - k (b.k)^T) X = X - k ((b.k)^T X). That is matrix associativity only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/*
 * One (sequence, value head) pair, tokens 0..T-1, all arrays row-major and
 * contiguous:
 *   q, k, log_alpha, b : [T][d_k]      v, w : [T][d_v]
 *   S                  : [d_k][d_v], holds S_0 on entry and S_T on return
 *   o                  : [T][d_v]
 * Returns 0, or -1 if scratch memory could not be allocated.
 */
int gdn2_oracle_sequence(int64_t T, int32_t d_k, int32_t d_v,
                         const double *q, const double *k,
                         const double *v, const double *w,
                         const double *log_alpha, const double *b,
                         double *S, double *o)
{
    double *y = (double *)malloc(sizeof(double) * (size_t)(d_v > 0 ? d_v : 1));
    if (!y) return -1;
    for (int64_t t = 0; t < T; ++t) {
        const double *qt = q + t * d_k, *kt = k + t * d_k;
        const double *lat = log_alpha + t * d_k, *bt = b + t * d_k;
        const double *vt = v + t * d_v, *wt = w + t * d_v;
        double *ot = o + t * d_v;

        /* decay: S <- diag(alpha_t) S, alpha on the key axis (rows) */
        for (int32_t i = 0; i < d_k; ++i) {
            double a = exp(lat[i]);
            for (int32_t j = 0; j < d_v; ++j) S[(size_t)i * d_v + j] *= a;
        }
        /* erase: S <- S - k_t ((b_t . k_t)^T S) */
        for (int32_t j = 0; j < d_v; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < d_k; ++i) acc += bt[i] * kt[i] * S[(size_t)i * d_v + j];
            y[j] = acc;
        }
        for (int32_t i = 0; i < d_k; ++i)
            for (int32_t j = 0; j < d_v; ++j) S[(size_t)i * d_v + j] -= kt[i] * y[j];
        /* write: S <- S + k_t (w_t . v_t)^T */
        for (int32_t i = 0; i < d_k; ++i)
            for (int32_t j = 0; j < d_v; ++j) S[(size_t)i * d_v + j] += kt[i] * (wt[j] * vt[j]);
        /* readout of the updated state: o_t = q_t^T S_t */
        for (int32_t j = 0; j < d_v; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < d_k; ++i) acc += qt[i] * S[(size_t)i * d_v + j];
            ot[j] = acc;
        }
    }
    free(y);
    return 0;
}

/*
 * Reverse-mode gradient of gdn2_oracle_sequence (same pair, same layouts), written from the
 * recurrence by the chain rule, one token at a time in reverse:
 *
 *   forward at token t:  S' = diag(a) S_{t-1},  a = exp(log_alpha_t),  s = b_t . k_t
 *                        u  = w_t . v_t - S'^T s,  S_t = S' + k_t u^T,  o_t = S_t^T q_t
 *   with G = dL/dS_t (starting from dS_T after the last token):
 *     G  += q_t do_t^T                     (o_t reads S_t)
 *     dq_t = S_t do_t
 *     du   = G^T k_t,        dk_t = G u + (-(S' du)) . b_t
 *     dw_t = du . v_t,       dv_t = du . w_t
 *     db_t = (-(S' du)) . k_t
 *     dS'  = G - s du^T      (y = S'^T s enters u with a minus sign)
 *     dlog_alpha_t = rowsum(dS' . S')      (S' = diag(exp(log_alpha)) S_{t-1})
 *     G    = diag(a) dS'     (dL/dS_{t-1})
 *   and dS0 = G at the end.
 *
 * The forward states are recomputed from checkpoints taken every CK tokens; within a
 * block of CK tokens they are kept, so memory is O(CK d_k d_v).
 *   do   : [T][d_v]        dST : [d_k][d_v] or NULL (zero)
 *   S0   : [d_k][d_v]      outputs dq, dk, dla, db : [T][d_k];  dv, dw : [T][d_v];  dS0
 * Returns 0, or -1 if scratch memory could not be allocated.
 */
int gdn2_oracle_sequence_bwd(int64_t T, int32_t d_k, int32_t d_v,
                             const double *q, const double *k,
                             const double *v, const double *w,
                             const double *log_alpha, const double *b,
                             const double *S0, const double *dout, const double *dST,
                             double *dq, double *dk, double *dv, double *dw,
                             double *dla, double *db, double *dS0)
{
    enum { CK = 64 };
    const size_t n = (size_t)d_k * d_v;
    const int64_t nblk = (T + CK - 1) / CK;
    double *ckpt = (double *)malloc(sizeof(double) * n * (size_t)(nblk > 0 ? nblk : 1));
    double *states = (double *)malloc(sizeof(double) * n * (CK + 1));
    double *G = (double *)malloc(sizeof(double) * n);
    double *Sp = (double *)malloc(sizeof(double) * n);
    double *u = (double *)malloc(sizeof(double) * (size_t)d_v);
    double *du = (double *)malloc(sizeof(double) * (size_t)d_v);
    double *sd = (double *)malloc(sizeof(double) * (size_t)d_k);
    if (!ckpt || !states || !G || !Sp || !u || !du || !sd) {
        free(ckpt); free(states); free(G); free(Sp); free(u); free(du); free(sd);
        return -1;
    }
    /* forward once, keeping the state entering every block */
    double *S = states;
    for (size_t e = 0; e < n; ++e) S[e] = S0[e];
    for (int64_t t = 0; t < T; ++t) {
        if (t % CK == 0)
            for (size_t e = 0; e < n; ++e) ckpt[(size_t)(t / CK) * n + e] = S[e];
        /* du serves as the (unused) output row of the forward step */
        gdn2_oracle_sequence(1, d_k, d_v, q + t * d_k, k + t * d_k, v + t * d_v, w + t * d_v,
                             log_alpha + t * d_k, b + t * d_k, S, du);
    }
    for (size_t e = 0; e < n; ++e) G[e] = dST ? dST[e] : 0.0;
    for (int64_t blk = nblk - 1; blk >= 0; --blk) {
        const int64_t t0 = blk * CK;
        const int64_t t1 = t0 + CK < T ? t0 + CK : T;
        /* states[j] = state entering token t0 + j; states[t1 - t0] = state after t1 - 1 */
        for (size_t e = 0; e < n; ++e) states[e] = ckpt[(size_t)blk * n + e];
        for (int64_t t = t0; t < t1; ++t) {
            double *dst = states + (size_t)(t - t0 + 1) * n;
            for (size_t e = 0; e < n; ++e) dst[e] = states[(size_t)(t - t0) * n + e];
            gdn2_oracle_sequence(1, d_k, d_v, q + t * d_k, k + t * d_k, v + t * d_v,
                                 w + t * d_v, log_alpha + t * d_k, b + t * d_k, dst, du);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double *Sprev = states + (size_t)(t - t0) * n;
            const double *St = states + (size_t)(t - t0 + 1) * n;
            const double *qt = q + t * d_k, *kt = k + t * d_k, *lat = log_alpha + t * d_k;
            const double *bt = b + t * d_k, *vt = v + t * d_v, *wt = w + t * d_v;
            const double *dot = dout + t * d_v;
            /* S' and u of the forward step */
            for (int32_t i = 0; i < d_k; ++i) {
                const double a = exp(lat[i]);
                for (int32_t j = 0; j < d_v; ++j) Sp[(size_t)i * d_v + j] = a * Sprev[(size_t)i * d_v + j];
            }
            for (int32_t j = 0; j < d_v; ++j) {
                double y = 0.0;
                for (int32_t i = 0; i < d_k; ++i) y += bt[i] * kt[i] * Sp[(size_t)i * d_v + j];
                u[j] = wt[j] * vt[j] - y;
            }
            /* G += q do^T ; dq = S_t do */
            for (int32_t i = 0; i < d_k; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < d_v; ++j) {
                    G[(size_t)i * d_v + j] += qt[i] * dot[j];
                    acc += St[(size_t)i * d_v + j] * dot[j];
                }
                dq[t * d_k + i] = acc;
            }
            /* du = G^T k */
            for (int32_t j = 0; j < d_v; ++j) {
                double acc = 0.0;
                for (int32_t i = 0; i < d_k; ++i) acc += G[(size_t)i * d_v + j] * kt[i];
                du[j] = acc;
                dw[t * d_v + j] = acc * vt[j];
                dv[t * d_v + j] = acc * wt[j];
            }
            /* sd = -(S' du): the gradient reaching s = b . k */
            for (int32_t i = 0; i < d_k; ++i) {
                double acc = 0.0, gu = 0.0;
                for (int32_t j = 0; j < d_v; ++j) {
                    acc += Sp[(size_t)i * d_v + j] * du[j];
                    gu += G[(size_t)i * d_v + j] * u[j];
                }
                sd[i] = -acc;
                db[t * d_k + i] = sd[i] * kt[i];
                dk[t * d_k + i] = gu + sd[i] * bt[i];
            }
            /* dS' = G - s du^T ; dlog_alpha = rowsum(dS' . S') ; G = diag(a) dS' */
            for (int32_t i = 0; i < d_k; ++i) {
                const double a = exp(lat[i]), s = bt[i] * kt[i];
                double acc = 0.0;
                for (int32_t j = 0; j < d_v; ++j) {
                    const double g = G[(size_t)i * d_v + j] - s * du[j];
                    acc += g * Sp[(size_t)i * d_v + j];
                    G[(size_t)i * d_v + j] = a * g;
                }
                dla[t * d_k + i] = acc;
            }
        }
    }
    for (size_t e = 0; e < n; ++e) dS0[e] = G[e];
    free(ckpt); free(states); free(G); free(Sp); free(u); free(du); free(sd);
    return 0;
}
