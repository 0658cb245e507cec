/*
 * fp64 CPU oracle for the Exact Flow Linear Attention (EFLA) operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or table with the HIP library.
 *
 * What it computes (source: "Exact Flow Linear Attention: Exact Solution from
 * Continuous-Time Dynamics", gist.science Technical Summary, Methodology 1-3):
 * the zero-order-hold ODE dS/dt = -k k^T S + k v^T, integrated exactly over a
 * token interval of length beta, gives the update
 *
 *     S_t = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T,
 *     alpha_t = (1 - exp(-beta_t lambda_t)) / lambda_t,   lambda_t = |k_t|^2,
 *
 * and the readout o_t = S_t^T q_t takes the state after the update.  At
 * lambda_t = 0 the formula for alpha is 0/0; its limit is beta_t, which is
 * also what the exponential collapses to when k_t = 0 (then kk^T = 0 and
 * the update is the identity whatever alpha is).
 *
 * With `euler` set, every function evaluates instead the explicit Euler step
 * of the same ODE over the interval beta, S + beta (-k k^T S + k v^T), i.e.
 * the same update with alpha_t = beta_t: the delta rule the pages compare the
 * exact flow against (Problem Statement; Methodology 3 calls the exact
 * update its continuous-time counterpart).
 *
 * The recurrence is evaluated token by token in fp64, one independent
 * (batch, head) sequence per OpenMP iteration.  (I - a k k^T) S is formed as
 * S - a k (k^T S): the same product, without materialising the d_k x d_k
 * matrix.  No chunking, no blocking, no reordering of the time loop.
 *
 * Layouts (row-major, contiguous):
 *   q, k [B,H,L,dk]   v, o [B,H,L,dv]   beta [B,H,L]   S0, S_L [B,H,dk,dv]
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* alpha_t from beta_t and lambda_t (Methodology 3, with the lambda -> 0 limit). */
double efla_oracle_alpha(double beta, double lambda)
{
    if (lambda == 0.0) return beta;
    return -expm1(-beta * lambda) / lambda;
}

/* One token: S <- (I - a k k^T) S + a k v^T, in place, a = alpha (or beta
 * for the Euler step).  kS is dv scratch. */
static void efla_oracle_token(double *S, const double *k, const double *v, double beta,
                              long dk, long dv, double *kS, int euler)
{
    double lambda = 0.0;
    for (long i = 0; i < dk; ++i) lambda += k[i] * k[i];
    const double a = euler ? beta : efla_oracle_alpha(beta, lambda);
    for (long j = 0; j < dv; ++j) kS[j] = 0.0;
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) kS[j] += k[i] * S[i * dv + j];
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) S[i * dv + j] += a * k[i] * (v[j] - kS[j]);
}

/* o = S^T q */
static void efla_oracle_readout(const double *S, const double *q, double *o, long dk, long dv)
{
    for (long j = 0; j < dv; ++j) o[j] = 0.0;
    for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) o[j] += S[i * dv + j] * q[i];
}

static int efla_oracle_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Whole-sequence forward.  S0 may be NULL (zero initial state).  Returns 0,
 * or -1 on a bad argument or failed scratch allocation.
 */
int efla_oracle_forward(const double *q, const double *k, const double *v, const double *beta,
                        const double *S0, double *o, double *S_L,
                        long B, long H, long L, long dk, long dv, int euler, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
    const long BH = B * H;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(efla_oracle_threads(nthreads))
    for (long bh = 0; bh < BH; ++bh) {
        double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!kS) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *S = S_L + bh * dk * dv;
        if (S0) memcpy(S, S0 + bh * dk * dv, sizeof(double) * (size_t)(dk * dv));
        else memset(S, 0, sizeof(double) * (size_t)(dk * dv));
        for (long t = 0; t < L; ++t) {
            const long tok = bh * L + t;
            efla_oracle_token(S, k + tok * dk, v + tok * dv, beta[tok], dk, dv, kS, euler);
            efla_oracle_readout(S, q + tok * dk, o + tok * dv, dk, dv);
        }
        free(kS);
    }
    return failed ? -1 : 0;
}

/*
 * One decode step for N sequences x H heads: S [N,H,dk,dv] is updated in
 * place and o [N,H,dv] = S_new^T q.  q, k [N,H,dk], v [N,H,dv], beta [N,H].
 */
int efla_oracle_decode(const double *q, const double *k, const double *v, const double *beta,
                       double *S, double *o, long N, long H, long dk, long dv, int euler,
                       int nthreads)
{
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    const long NH = N * H;
    int failed = 0;
#pragma omp parallel for schedule(static) num_threads(efla_oracle_threads(nthreads))
    for (long nh = 0; nh < NH; ++nh) {
        double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!kS) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *Sh = S + nh * dk * dv;
        efla_oracle_token(Sh, k + nh * dk, v + nh * dv, beta[nh], dk, dv, kS, euler);
        efla_oracle_readout(Sh, q + nh * dk, o + nh * dv, dk, dv);
        free(kS);
    }
    return failed ? -1 : 0;
}

/* Number of threads an OpenMP region would use (for reporting). */
int efla_oracle_max_threads(void)
{
    return efla_oracle_threads(0);
}
