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

/* ---------------------------------------------------------------------------
 * Reverse mode of eqs (1)-(4): gradients of a scalar loss L whose partial
 * derivatives with respect to the outputs are given, dL/dy_t = dy_t for every
 * token and dL/dS_T = dST (NULL: zero).  Per (b, h) the token steps are undone
 * in reverse order; step t, entered with dS = dL/dS_t (everything after token
 * t already folded in), applies the chain rule to each of (4), (3), (2), (1):
 *
 *   (4) y_t = S_t^T q_t          dS += q_t dy_t^T;   dq_t = S_t dy_t
 *   (3) S_t = S~ + beta k e^T    dbeta_t = k^T dS e;  de = beta dS^T k;
 *                                dk_t = beta dS e;    dS~ = dS
 *   (2) e = v - S~^T k           dv_t = de;  dk_t -= S~ de;  dS~ -= k de^T
 *   (1) S~ = alpha S_{t-1}       dalpha_t = <S_{t-1}, dS~>;  dS = alpha dS~
 *
 * and after token 0, dS0 = dS.  S_{t-1} is needed in reverse order: the states
 * entering every SEG-th token are kept on the way forward and each segment's
 * states are recomputed from its checkpoint, in the same token steps as the
 * forward loop above.
 *
 * Layouts as above; dq, dk like q; dv, dy like v; dalpha, dbeta like alpha;
 * dS0, dST like S0.  Returns 0, or -1 on allocation failure.
 * ------------------------------------------------------------------------- */
#define BWD_SEG 64

int oracle_gdn_recurrence_bwd(const double *q, const double *k, const double *v,
                              const double *alpha, const double *beta, const double *S0,
                              const double *dy, const double *dST,
                              double *dq, double *dk, double *dv, double *dalpha,
                              double *dbeta, double *dS0,
                              int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                              int nthreads, int *threads_used)
{
    const int nt = set_threads(nthreads);
    const int64_t SS = Dk * Dv;
    const int64_t nseg = (T + BWD_SEG - 1) / BWD_SEG;
    int failed = 0;
    int used = 1;
    #pragma omp parallel num_threads(nt)
    {
        #ifdef _OPENMP
        #pragma omp single
        used = omp_get_num_threads();
        #endif
        /* ck: state entering token s*SEG for every segment s;
         * prev: state entering each token of the current segment */
        double *ck   = (double *)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * SS));
        double *prev = (double *)malloc(sizeof(double) * (size_t)(BWD_SEG * SS));
        double *S    = (double *)malloc(sizeof(double) * (size_t)SS);
        double *St   = (double *)malloc(sizeof(double) * (size_t)SS);
        double *dS   = (double *)malloc(sizeof(double) * (size_t)SS);
        double *e    = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *de   = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *yt   = (double *)malloc(sizeof(double) * (size_t)Dv);
        const int ok = ck && prev && S && St && dS && e && de && yt;
        if (!ok) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (!ok) continue;
            const int64_t b = bh / H, h = bh % H;

            /* forward, keeping a checkpoint at the start of every segment */
            if (S0) memcpy(S, S0 + bh * SS, sizeof(double) * (size_t)SS);
            else    memset(S, 0, sizeof(double) * (size_t)SS);
            for (int64_t t = 0; t < T; ++t) {
                if (t % BWD_SEG == 0) memcpy(ck + (t / BWD_SEG) * SS, S, sizeof(double) * (size_t)SS);
                const int64_t row = (b * T + t) * H + h;
                gated_delta_token(S, St, e, q + row * Dk, k + row * Dk, v + row * Dv,
                                  alpha[row], beta[row], yt, Dk, Dv);
            }

            if (dST) memcpy(dS, dST + bh * SS, sizeof(double) * (size_t)SS);
            else     memset(dS, 0, sizeof(double) * (size_t)SS);

            for (int64_t s = nseg - 1; s >= 0; --s) {
                const int64_t t0 = s * BWD_SEG;
                const int64_t t1 = t0 + BWD_SEG < T ? t0 + BWD_SEG : T;
                /* states entering tokens t0..t1-1 */
                memcpy(S, ck + s * SS, sizeof(double) * (size_t)SS);
                for (int64_t t = t0; t < t1; ++t) {
                    memcpy(prev + (t - t0) * SS, S, sizeof(double) * (size_t)SS);
                    const int64_t row = (b * T + t) * H + h;
                    gated_delta_token(S, St, e, q + row * Dk, k + row * Dk, v + row * Dv,
                                      alpha[row], beta[row], yt, Dk, Dv);
                }
                for (int64_t t = t1 - 1; t >= t0; --t) {
                    const int64_t row = (b * T + t) * H + h;
                    const double *qt = q + row * Dk, *kt = k + row * Dk, *vt = v + row * Dv;
                    const double *dyt = dy + row * Dv;
                    const double *Sp = prev + (t - t0) * SS;
                    const double a = alpha[row], bt = beta[row];

                    /* recompute S~, e and S_t of this token */
                    for (int64_t i = 0; i < SS; ++i) St[i] = a * Sp[i];
                    for (int64_t j = 0; j < Dv; ++j) {
                        double pred = 0.0;
                        for (int64_t i = 0; i < Dk; ++i) pred += St[i * Dv + j] * kt[i];
                        e[j] = vt[j] - pred;
                    }
                    for (int64_t i = 0; i < Dk; ++i)
                        for (int64_t j = 0; j < Dv; ++j)
                            S[i * Dv + j] = St[i * Dv + j] + bt * kt[i] * e[j];

                    /* (4) */
                    for (int64_t i = 0; i < Dk; ++i) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < Dv; ++j) acc += S[i * Dv + j] * dyt[j];
                        dq[row * Dk + i] = acc;
                    }
                    for (int64_t i = 0; i < Dk; ++i)
                        for (int64_t j = 0; j < Dv; ++j)
                            dS[i * Dv + j] += qt[i] * dyt[j];

                    /* (3) */
                    double db = 0.0;
                    for (int64_t i = 0; i < Dk; ++i)
                        for (int64_t j = 0; j < Dv; ++j)
                            db += kt[i] * dS[i * Dv + j] * e[j];
                    dbeta[row] = db;
                    for (int64_t j = 0; j < Dv; ++j) {
                        double acc = 0.0;
                        for (int64_t i = 0; i < Dk; ++i) acc += dS[i * Dv + j] * kt[i];
                        de[j] = bt * acc;
                    }
                    for (int64_t i = 0; i < Dk; ++i) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < Dv; ++j) acc += dS[i * Dv + j] * e[j];
                        dk[row * Dk + i] = bt * acc;
                    }

                    /* (2) */
                    for (int64_t j = 0; j < Dv; ++j) dv[row * Dv + j] = de[j];
                    for (int64_t i = 0; i < Dk; ++i) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < Dv; ++j) acc += St[i * Dv + j] * de[j];
                        dk[row * Dk + i] -= acc;
                    }
                    for (int64_t i = 0; i < Dk; ++i)
                        for (int64_t j = 0; j < Dv; ++j)
                            dS[i * Dv + j] -= kt[i] * de[j];

                    /* (1) */
                    double da = 0.0;
                    for (int64_t i = 0; i < SS; ++i) da += Sp[i] * dS[i];
                    dalpha[row] = da;
                    for (int64_t i = 0; i < SS; ++i) dS[i] *= a;
                }
            }
            if (dS0) memcpy(dS0 + bh * SS, dS, sizeof(double) * (size_t)SS);
        }
        free(ck); free(prev); free(S); free(St); free(dS); free(e); free(de); free(yt);
    }
    if (threads_used) *threads_used = used;
    return failed ? -1 : 0;
}
