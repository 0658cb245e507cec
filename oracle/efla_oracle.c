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

/*
 * Partial derivatives of alpha(beta, lambda) (Methodology 3's coefficient):
 * with x = beta lambda, alpha = (1 - e^{-x}) / lambda, so
 *     d alpha / d beta   = e^{-x},
 *     d alpha / d lambda = (x e^{-x} - (1 - e^{-x})) / lambda^2 = -beta^2 g(x),
 *     g(x) = (1 - (1 + x) e^{-x}) / x^2 = sum_{n>=0} (-1)^n (n+1) x^n / (n+2)!,
 * g(0) = 1/2 (the lambda -> 0 limit, where alpha -> beta).  The series is
 * summed for |x| < 1/2 (the closed form cancels there), the closed form
 * otherwise.  Euler: alpha = beta, so the derivatives are 1 and 0.
 */
void efla_oracle_alpha_grad(double beta, double lambda, int euler, double *da_dbeta,
                            double *da_dlambda)
{
    if (euler) {
        *da_dbeta = 1.0;
        *da_dlambda = 0.0;
        return;
    }
    const double x = beta * lambda;
    double g;
    if (fabs(x) < 0.5) {
        double term = 0.5, sum = 0.0;   /* term_n = (-1)^n (n+1) x^n / (n+2)! */
        for (int n = 0; n < 30; ++n) {
            sum += term;
            term *= -x * (double)(n + 2) / ((double)(n + 1) * (double)(n + 3));
        }
        g = sum;
    } else {
        g = (-expm1(-x) - x * exp(-x)) / (x * x);
    }
    *da_dbeta = exp(-x);
    *da_dlambda = -beta * beta * g;
}

/*
 * Gradients of a scalar loss through the whole-sequence forward, given
 * dO = dLoss/do [B,H,L,dv] and dS_L = dLoss/dS_L [B,H,dk,dv] (NULL = 0):
 * dq, dk [B,H,L,dk], dv [B,H,L,dv], dbeta [B,H,L], dS0 [B,H,dk,dv].
 *
 * The adjoint of the token recurrence, run backwards in time.  With
 * r_t = v_t - S_{t-1}^T k_t, e_t = alpha_t r_t, S_t = S_{t-1} + k_t e_t^T and
 * o_t = S_t^T q_t, and G = dLoss/dS_t accumulated from the later tokens:
 *     G      += q_t do_t^T                  dq_t = S_t do_t
 *     de      = G^T k_t                     dk_t = G e_t
 *     dalpha  = de . r_t                    dr   = alpha_t de = dv_t
 *     dk_t   -= S_{t-1} dr                  G    -= k_t dr^T   (now dLoss/dS_{t-1})
 *     dbeta_t = dalpha dalpha/dbeta         dk_t += 2 dalpha dalpha/dlambda k_t
 * and dS0 is G after token 0.  The states S_t the adjoint needs are
 * recomputed by the same token update from a copy of S taken every 64
 * tokens (identical values to keeping them all; only memory differs).
 */
int efla_oracle_backward(const double *q, const double *k, const double *v, const double *beta,
                         const double *S0, const double *dO, const double *dSL, double *dq,
                         double *dk_out, double *dv_out, double *dbeta, double *dS0,
                         long B, long H, long L, long dk, long dv, int euler, int nthreads)
{
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
    const long BH = B * H, CK = 64, nck = (L + CK - 1) / CK, SZ = dk * dv;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(efla_oracle_threads(nthreads))
    for (long bh = 0; bh < BH; ++bh) {
        double *ck = (double *)malloc(sizeof(double) * (size_t)((nck + 1) * SZ));
        double *blk = (double *)malloc(sizeof(double) * (size_t)((CK + 1) * SZ));
        double *G = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *tmp = (double *)malloc(sizeof(double) * (size_t)(3 * dv));
        if (!ck || !blk || !G || !tmp) {
            free(ck); free(blk); free(G); free(tmp);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *kS = tmp, *de = tmp + dv, *r = tmp + 2 * dv;
        /* forward, keeping S before tokens 0, 64, 128, ... */
        double *S = blk;
        if (S0) memcpy(S, S0 + bh * SZ, sizeof(double) * (size_t)SZ);
        else memset(S, 0, sizeof(double) * (size_t)SZ);
        for (long t = 0; t < L; ++t) {
            if (t % CK == 0) memcpy(ck + (t / CK) * SZ, S, sizeof(double) * (size_t)SZ);
            const long tok = bh * L + t;
            efla_oracle_token(S, k + tok * dk, v + tok * dv, beta[tok], dk, dv, kS, euler);
        }
        if (L == 0) memcpy(ck, S, sizeof(double) * (size_t)SZ);
        if (dSL) memcpy(G, dSL + bh * SZ, sizeof(double) * (size_t)SZ);
        else memset(G, 0, sizeof(double) * (size_t)SZ);

        for (long b = nck - 1; b >= 0; --b) {
            const long t0 = b * CK, t1 = (t0 + CK < L) ? t0 + CK : L;
            /* blk[j] = S_{t0 + j - 1}: the state before token t0 + j */
            memcpy(blk, ck + b * SZ, sizeof(double) * (size_t)SZ);
            for (long t = t0; t < t1; ++t) {
                double *nxt = blk + (t - t0 + 1) * SZ;
                memcpy(nxt, blk + (t - t0) * SZ, sizeof(double) * (size_t)SZ);
                const long tok = bh * L + t;
                efla_oracle_token(nxt, k + tok * dk, v + tok * dv, beta[tok], dk, dv, kS, euler);
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const long tok = bh * L + t;
                const double *Sp = blk + (t - t0) * SZ, *Sc = blk + (t - t0 + 1) * SZ;
                const double *kt = k + tok * dk, *vt = v + tok * dv, *qt = q + tok * dk;
                const double *dot = dO + tok * dv;
                double *dqt = dq + tok * dk, *dkt = dk_out + tok * dk, *dvt = dv_out + tok * dv;
                double lambda = 0.0;
                for (long i = 0; i < dk; ++i) lambda += kt[i] * kt[i];
                const double a = euler ? beta[tok] : efla_oracle_alpha(beta[tok], lambda);
                /* r = v - S_{t-1}^T k */
                for (long j = 0; j < dv; ++j) r[j] = vt[j];
                for (long i = 0; i < dk; ++i)
                    for (long j = 0; j < dv; ++j) r[j] -= Sp[i * dv + j] * kt[i];
                /* readout o_t = S_t^T q_t */
                for (long i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < dv; ++j) {
                        G[i * dv + j] += qt[i] * dot[j];
                        acc += Sc[i * dv + j] * dot[j];
                    }
                    dqt[i] = acc;
                }
                /* S_t = S_{t-1} + k e^T, e = a r */
                for (long j = 0; j < dv; ++j) de[j] = 0.0;
                for (long i = 0; i < dk; ++i)
                    for (long j = 0; j < dv; ++j) de[j] += G[i * dv + j] * kt[i];
                for (long i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < dv; ++j) acc += G[i * dv + j] * a * r[j];
                    dkt[i] = acc;
                }
                double dalpha = 0.0;
                for (long j = 0; j < dv; ++j) dalpha += de[j] * r[j];
                /* e = a (v - S_{t-1}^T k) */
                for (long j = 0; j < dv; ++j) dvt[j] = a * de[j];
                for (long i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (long j = 0; j < dv; ++j) {
                        acc += Sp[i * dv + j] * dvt[j];
                        G[i * dv + j] -= kt[i] * dvt[j];
                    }
                    dkt[i] -= acc;
                }
                /* alpha = alpha(beta, |k|^2) */
                double da_db, da_dl;
                efla_oracle_alpha_grad(beta[tok], lambda, euler, &da_db, &da_dl);
                dbeta[tok] = dalpha * da_db;
                for (long i = 0; i < dk; ++i) dkt[i] += 2.0 * dalpha * da_dl * kt[i];
            }
        }
        memcpy(dS0 + bh * SZ, G, sizeof(double) * (size_t)SZ);
        free(ck); free(blk); free(G); free(tmp);
    }
    return failed ? -1 : 0;
}

/* Number of threads an OpenMP region would use (for reporting). */
int efla_oracle_max_threads(void)
{
    return efla_oracle_threads(0);
}
