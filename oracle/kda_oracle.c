/*
 * KDA forward oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation of the Kimi Delta
 * Attention (gated delta rule with per-channel decay) forward pass, in fp64.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code with the GPU library.
 *
 * What it computes (KDA TPU report, section 1 and section 2: the recurrence
 * with a fixed-size [K, V] state per head; section 6.5: packed varlen
 * sequences with an optional initial state per sequence).  For every
 * sequence s (tokens cu[s] .. cu[s+1]-1) and head h, independently:
 *
 *     S   <- initial_state[s, h]  (or 0)                  S is [dk, dv]
 *     for each token t in order:
 *         S   <- Diag(exp(g_t)) S                         per-key-channel decay
 *         S   <- S + beta_t k_t (v_t - S^T k_t)^T         delta-rule write
 *         o_t <- scale * S^T q_t                          reads the updated S
 *     final_state[s, h] <- S
 *
 * The write step is (I - beta k k^T) Diag(exp g) S + beta k v^T expanded.
 * Inputs arrive as fp32 (bf16 values widen exactly); all arithmetic is fp64
 * with libm exp.  OpenMP splits the independent (sequence, head) pairs and
 * does not change any result.
 *
 * Layouts (row-major, contiguous):
 *   q, k, g   [T, H, dk]      v, o  [T, H, dv]      beta [T, H]
 *   initial_state, final_state [N, H, dk, dv]      cu_seqlens [N+1]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, nonzero on a malformed cu_seqlens or bad sizes. */
int kda_oracle_fwd(const float *q, const float *k, const float *v,
                   const float *g, const float *beta,
                   const float *initial_state, const int32_t *cu_seqlens,
                   int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                   double scale, double *o, double *final_state,
                   int32_t nthreads)
{
    if (T < 0 || N < 1 || H < 1 || dk < 1 || dv < 1) return 1;
    if (cu_seqlens[0] != 0 || (int64_t)cu_seqlens[N] != T) return 2;
    for (int32_t s = 0; s < N; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return 3;

    const int64_t pairs = (int64_t)N * H;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t p = 0; p < pairs; ++p) {
        const int32_t s = (int32_t)(p / H);
        const int32_t h = (int32_t)(p % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !u) { free(S); free(u); bad |= 1; continue; }
        const size_t st_off = ((size_t)s * H + h) * (size_t)dk * dv;
        for (int64_t e = 0; e < (int64_t)dk * dv; ++e)
            S[e] = initial_state ? (double)initial_state[st_off + e] : 0.0;

        for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
            const float *qt = q + ((size_t)t * H + h) * dk;
            const float *kt = k + ((size_t)t * H + h) * dk;
            const float *gt = g + ((size_t)t * H + h) * dk;
            const float *vt = v + ((size_t)t * H + h) * dv;
            const double bt = (double)beta[(size_t)t * H + h];

            /* decay: row i of S (key channel i) scales by exp(g_t[i]) */
            for (int32_t i = 0; i < dk; ++i) {
                const double a = exp((double)gt[i]);
                double *row = S + (size_t)i * dv;
                for (int32_t j = 0; j < dv; ++j) row[j] *= a;
            }
            /* u = S^T k  (what the decayed state predicts for key k_t) */
            for (int32_t j = 0; j < dv; ++j) u[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i) {
                const double ki = (double)kt[i];
                const double *row = S + (size_t)i * dv;
                for (int32_t j = 0; j < dv; ++j) u[j] += ki * row[j];
            }
            /* u <- beta (v - u); S <- S + k u^T */
            for (int32_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - u[j]);
            for (int32_t i = 0; i < dk; ++i) {
                const double ki = (double)kt[i];
                double *row = S + (size_t)i * dv;
                for (int32_t j = 0; j < dv; ++j) row[j] += ki * u[j];
            }
            /* o_t = scale * S^T q_t */
            double *ot = o + ((size_t)t * H + h) * dv;
            for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int32_t i = 0; i < dk; ++i) {
                const double qi = (double)qt[i];
                const double *row = S + (size_t)i * dv;
                for (int32_t j = 0; j < dv; ++j) ot[j] += qi * row[j];
            }
            for (int32_t j = 0; j < dv; ++j) ot[j] *= scale;
        }
        if (final_state)
            memcpy(final_state + st_off, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(u);
    }
    return bad ? 4 : 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int32_t kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
