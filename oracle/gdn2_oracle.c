/*
 * gdn2_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU evaluation of the Gated DeltaNet-2 recurrence. It exists
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
 *     no index; the llama.cpp decode notes, section 2, read out after the rank-1
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
