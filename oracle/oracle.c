/*
 * oracle.c -- plain, slow, fp64 CPU implementation of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the GPU library
 * is checked against.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no source, header,
 * helper or constant with the HIP library and includes no GPU header.
 *
 * What it computes (source: "On the Design of Qwen3.8-Next Architecture",
 * picx.dev summary page, section "Theoretical foundations", eqs (1)-(4)):
 * for every (batch b, head h) independently, with state S in R^{Dk x Dv},
 *
 *     S~_{t-1} = alpha_t * S_{t-1}                       (1)
 *     e_t      = v_t - S~_{t-1}^T k_t                     (2)
 *     S_t      = S~_{t-1} + beta_t * k_t e_t^T            (3)
 *     y_t      = S_t^T q_t                                (4)
 *
 * The loop below takes these four steps in this order, token by token, in
 * double precision, with no blocking, fusion or reordering.  Nothing is
 * rounded between steps.
 *
 * Layouts (row-major, last index fastest):
 *   q, k   : [B, T, H, Dk]
 *   v, y   : [B, T, H, Dv]
 *   alpha, beta : [B, T, H]
 *   S0, ST : [B, H, Dk, Dv]   (S0 may be NULL: zero initial state)
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of eqs (1)-(4) for one head.
 * S    : Dk x Dv state, updated in place (becomes S_t)
 * St   : Dk x Dv scratch for S~_{t-1}
 * e    : Dv scratch
 * y    : Dv output, y_t = S_t^T q_t                                        */
static void gated_delta_token(double *S, double *St, double *e,
                              const double *q, const double *k, const double *v,
                              double alpha, double beta, double *y,
                              int64_t Dk, int64_t Dv)
{
    /* (1) decayed state */
    for (int64_t i = 0; i < Dk; ++i)
        for (int64_t j = 0; j < Dv; ++j)
            St[i * Dv + j] = alpha * S[i * Dv + j];

    /* (2) error of the decayed state's prediction for key k_t */
    for (int64_t j = 0; j < Dv; ++j) {
        double pred = 0.0;
        for (int64_t i = 0; i < Dk; ++i)
            pred += St[i * Dv + j] * k[i];
        e[j] = v[j] - pred;
    }

    /* (3) rank-one write of the error */
    for (int64_t i = 0; i < Dk; ++i)
        for (int64_t j = 0; j < Dv; ++j)
            S[i * Dv + j] = St[i * Dv + j] + beta * k[i] * e[j];

    /* (4) read-out from the updated state */
    for (int64_t j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < Dk; ++i)
            acc += S[i * Dv + j] * q[i];
        y[j] = acc;
    }
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) return nthreads;
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Whole-sequence recurrence: every (b, h) runs eqs (1)-(4) for t = 0..T-1.
 * Returns 0 on success, -1 on allocation failure.  `nthreads` <= 0 means the
 * OpenMP default; the number actually used is written to *threads_used.   */
int oracle_gdn_recurrence(const double *q, const double *k, const double *v,
                          const double *alpha, const double *beta,
                          const double *S0, double *y, double *ST,
                          int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                          int nthreads, int *threads_used)
{
    const int nt = set_threads(nthreads);
    int failed = 0;
    int used = 1;
    #pragma omp parallel num_threads(nt)
    {
        #ifdef _OPENMP
        #pragma omp single
        used = omp_get_num_threads();
        #endif
        double *S  = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *St = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *e  = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!S || !St || !e) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (!S || !St || !e) continue;
            const int64_t b = bh / H, h = bh % H;
            if (S0) memcpy(S, S0 + bh * Dk * Dv, sizeof(double) * (size_t)(Dk * Dv));
            else    memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = (b * T + t) * H + h;
                gated_delta_token(S, St, e, q + row * Dk, k + row * Dk, v + row * Dv,
                                  alpha[row], beta[row], y + row * Dv, Dk, Dv);
            }
            if (ST) memcpy(ST + bh * Dk * Dv, S, sizeof(double) * (size_t)(Dk * Dv));
        }
        free(S); free(St); free(e);
    }
    if (threads_used) *threads_used = used;
    return failed ? -1 : 0;
}

/* One recurrent step for N independent sequences: the same per-token update
 * applied once to each state, which is updated in place.
 * q, k : [N, H, Dk]; v, y : [N, H, Dv]; alpha, beta : [N, H];
 * S    : [N, H, Dk, Dv].                                                    */
int oracle_gdn_decode_step(const double *q, const double *k, const double *v,
                           const double *alpha, const double *beta,
                           double *S, double *y,
                           int64_t N, int64_t H, int64_t Dk, int64_t Dv,
                           int nthreads, int *threads_used)
{
    const int nt = set_threads(nthreads);
    int failed = 0;
    int used = 1;
    #pragma omp parallel num_threads(nt)
    {
        #ifdef _OPENMP
        #pragma omp single
        used = omp_get_num_threads();
        #endif
        double *St = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *e  = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!St || !e) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(static)
        for (int64_t nh = 0; nh < N * H; ++nh) {
            if (!St || !e) continue;
            gated_delta_token(S + nh * Dk * Dv, St, e, q + nh * Dk, k + nh * Dk,
                              v + nh * Dv, alpha[nh], beta[nh], y + nh * Dv, Dk, Dv);
        }
        free(St); free(e);
    }
    if (threads_used) *threads_used = used;
    return failed ? -1 : 0;
}
