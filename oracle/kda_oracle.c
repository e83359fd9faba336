/*
 * kda_oracle.c -- plain, slow, fp64 CPU oracle for the Kimi Delta Attention
 * (KDA) gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes (sources: the dev.to page "Kimi K3 Architecture: Scaling
 * 2.8T Parameters for Long-Context Multimodal MoE", section "The Sequence
 * Bottleneck: Hybrid KDA and Gated MLA", with its gate equation; the
 * terrencekim.net page "Kimi K3 - Sparsity Mechanics ...", section 2
 * "Multi-Tiered Token & Memory Compression Engine", Temporal Sequence card):
 *
 *   per head a state S in R^{dk x dv}; row index = key channel.
 *   gate      g_t   = g_min * sigmoid(exp(A_h) * z_t)        (elementwise, dk)
 *   retention a_t   = exp(g_t)                                in (e^g_min, 1)
 *   update    S_t   = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T
 *   output    o_t   = S_t^T q_t
 *
 * The pages describe the update only in words (delta rule, Householder-style
 * erase, channel-wise forget gate); the algebraic form above -- decay first,
 * then the rank-one erase and write, output from the updated state, no 1/sqrt(d)
 * scale -- is the reading this oracle implements.
 *
 * Everything internal is double.  Inputs arrive as float32 arrays holding the
 * exact values the GPU saw (bf16 and fp32 both widen exactly), and are widened
 * to double on read.  Outputs are double.
 *
 * Layouts (contiguous, row-major):
 *   q, k, z : [B, T, H, dk]        v, o : [B, T, H, dv]
 *   beta    : [B, T, H]            A    : [H]
 *   S0, S_T : [B, H, dk, dv]       (S0 may be NULL: zeros)
 * Decode uses the same layouts with T = 1 and the state updated in place.
 *
 * Parallelism: one (b, h) pair per OpenMP task; nothing else is reordered.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Logistic function 1 / (1 + e^{-x}), evaluated through whichever of its two
 * equal forms cannot overflow. */
static double logistic(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* Lower-bounded log-decay g = g_min * Sigmoid(e^{A_h} z), per key channel
 * (dev.to page, gate equation in "The Sequence Bottleneck"). */
static double log_decay(double z, double a_h, double g_min)
{
    return g_min * logistic(exp(a_h) * z);
}

/* g for every element of z: g[b,t,h,c]. */
void kda_oracle_gate(const float *z, const float *A, double g_min,
                     long B, long T, long H, long dk, double *g)
{
    for (long b = 0; b < B; ++b)
        for (long t = 0; t < T; ++t)
            for (long h = 0; h < H; ++h) {
                size_t base = (((size_t)b * T + t) * H + h) * dk;
                for (long c = 0; c < dk; ++c)
                    g[base + c] = log_decay(z[base + c], A[h], g_min);
            }
}

/* Chunk-local cumulative log-decay: within each block of C consecutive tokens
 * starting at t = 0, C, 2C, ... the inclusive running sum of g restarts.
 * (dev.to page: the 16-token tiles whose cumulative log-decay the lower bound
 * keeps inside (-80, 0).)  G has the layout of z. */
void kda_oracle_gate_chunk_cumsum(const float *z, const float *A, double g_min,
                                  long B, long T, long H, long dk, long C,
                                  double *G)
{
    for (long b = 0; b < B; ++b)
        for (long h = 0; h < H; ++h)
            for (long c = 0; c < dk; ++c) {
                double run = 0.0;
                for (long t = 0; t < T; ++t) {
                    if (t % C == 0)
                        run = 0.0;
                    size_t i = (((size_t)b * T + t) * H + h) * dk + c;
                    run += log_decay(z[i], A[h], g_min);
                    G[i] = run;
                }
            }
}

/* One token of the recurrence on one head's state S[dk][dv] (in place).
 * qv, kv, zv: dk values; vv: dv values; writes dv outputs to out. */
static void step_one_token(long dk, long dv, double *S, const float *qv,
                           const float *kv, const float *vv, const float *zv,
                           double beta, double a_h, double g_min, double *out,
                           double *scratch /* dk + dv */)
{
    double *alpha = scratch;      /* dk */
    double *erase = scratch + dk; /* dv: k^T Diag(alpha) S_{t-1} */

    /* Diag(alpha_t) S_{t-1}: scale each key-channel row. */
    for (long c = 0; c < dk; ++c) {
        alpha[c] = exp(log_decay(zv[c], a_h, g_min));
        for (long j = 0; j < dv; ++j)
            S[c * dv + j] *= alpha[c];
    }
    /* (I - beta k k^T) S' + beta k v^T  =  S' + k (beta (v - S'^T k))^T */
    for (long j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (long c = 0; c < dk; ++c)
            acc += (double)kv[c] * S[c * dv + j];
        erase[j] = acc;
    }
    for (long c = 0; c < dk; ++c) {
        double kc = kv[c];
        for (long j = 0; j < dv; ++j)
            S[c * dv + j] += kc * beta * ((double)vv[j] - erase[j]);
    }
    /* o_t = S_t^T q_t */
    for (long j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (long c = 0; c < dk; ++c)
            acc += (double)qv[c] * S[c * dv + j];
        out[j] = acc;
    }
}

/* Token-by-token prefill over T tokens for every (b, h).  S_T may be NULL. */
int kda_oracle_prefill(const float *q, const float *k, const float *v,
                       const float *z, const float *beta, const float *A,
                       double g_min, const float *S0, double *o, double *S_T,
                       long B, long T, long H, long dk, long dv, int nthreads)
{
    long units = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|| : failed)
#endif
    for (long u = 0; u < units; ++u) {
        long b = u / H, h = u % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv + dk + dv));
        if (!S) {
            failed = 1;
            continue;
        }
        double *scratch = S + dk * dv;
        size_t sbase = ((size_t)b * H + h) * (size_t)(dk * dv);
        for (long e = 0; e < dk * dv; ++e)
            S[e] = S0 ? (double)S0[sbase + e] : 0.0;
        for (long t = 0; t < T; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            step_one_token(dk, dv, S, q + row * dk, k + row * dk, v + row * dv,
                           z + row * dk, beta[row], A[h], g_min, o + row * dv,
                           scratch);
        }
        if (S_T)
            for (long e = 0; e < dk * dv; ++e)
                S_T[sbase + e] = S[e];
        free(S);
    }
    return failed ? 1 : 0;
}

/* One decode step for every (b, h): inputs [B, H, d], beta [B, H], state
 * S [B, H, dk, dv] updated in place (double), outputs o [B, H, dv]. */
int kda_oracle_decode(const float *q, const float *k, const float *v,
                      const float *z, const float *beta, const float *A,
                      double g_min, double *S, double *o, long B, long H,
                      long dk, long dv, int nthreads)
{
    long units = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads) reduction(|| : failed)
#endif
    for (long u = 0; u < units; ++u) {
        long h = u % H;
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(dk + dv));
        if (!scratch) {
            failed = 1;
            continue;
        }
        step_one_token(dk, dv, S + (size_t)u * (size_t)(dk * dv), q + (size_t)u * dk,
                       k + (size_t)u * dk, v + (size_t)u * dv, z + (size_t)u * dk,
                       beta[u], A[h], g_min, o + (size_t)u * dv, scratch);
        free(scratch);
    }
    return failed ? 1 : 0;
}

/* Gradients of the token-by-token prefill (reverse-mode differentiation of
 * the recurrence above, written out step by step; the pages describe no
 * backward pass, so this is the exact gradient of the forward definition).
 *
 * Scalar loss: L = sum(dO * o) + sum(dST * S_T), i.e. dO and dST are the
 * incoming gradients of o and S_T (dST may be NULL: zeros).  Outputs (double):
 *   dq, dk, dz [B,T,H,dk], dv [B,T,H,dv], dbeta [B,T,H], dA [H],
 *   dS0 [B,H,dk,dv] (the gradient of the initial state, whether or not S0 is
 *   NULL).
 * Every per-token state S_0 .. S_T of a head is kept (T+1 copies of dk x dv
 * doubles), so this is for small and medium T.
 *
 * Per token (forward, for reference):
 *   x = e^{A} z, s = Sigmoid(x), a = e^{g_min s}, S' = Diag(a) S_{t-1},
 *   u = v - S'^T k, e = beta u, S_t = S' + k e^T, o = S_t^T q.
 * Reverse, with dS the gradient of S_t (dST at t = T-1):
 *   dS += q do^T;         dq = S_t do
 *   de = dS^T k;          dk = dS e;       dbeta = de . u;   dv = beta de
 *   dp = -beta de;        dS' = dS + k dp^T;   dk += S' dp
 *   da = rowsum(dS' o S_{t-1});   dg = da a;   dx = dg g_min s (1 - s)
 *   dz = dx e^{A};        dA += dx x;      dS_{t-1} = Diag(a) dS'
 */
int kda_oracle_backward(const float *q, const float *k, const float *v,
                        const float *z, const float *beta, const float *A,
                        double g_min, const float *S0, const float *dO,
                        const float *dST, double *dq, double *dk, double *dv,
                        double *dz, double *dbeta, double *dA, double *dS0,
                        long B, long T, long H, long dk_, long dv_, int nthreads)
{
    const long DK = dk_, DV = dv_, units = B * H;
    const size_t SS = (size_t)DK * DV;
    double *dA_unit = (double *)calloc((size_t)units, sizeof(double));
    if (!dA_unit)
        return 1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads < 1)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(|| : failed)
#endif
    for (long u = 0; u < units; ++u) {
        const long b = u / H, h = u % H;
        /* states S_0 .. S_T, per token: a, s, x (dk each), u (dv) */
        double *St = (double *)malloc(sizeof(double) * (SS * (size_t)(T + 1)));
        double *tok = (double *)malloc(sizeof(double) * ((size_t)T * (3 * DK + DV) + 2 * SS + DK + DV));
        if (!St || !tok) {
            free(St);
            free(tok);
            failed = 1;
            continue;
        }
        double *dS = tok + (size_t)T * (3 * DK + DV);
        double *dSp = dS + SS;
        double *de = dSp + SS; /* dv */
        double *da = de + DV;  /* dk */
        const double eA = exp((double)A[h]);
        const size_t sbase = ((size_t)b * H + h) * SS;
        for (size_t e = 0; e < SS; ++e)
            St[e] = S0 ? (double)S0[sbase + e] : 0.0;
        /* forward, keeping what the reverse sweep needs */
        for (long t = 0; t < T; ++t) {
            const size_t row = ((size_t)b * T + t) * H + h;
            const float *kv = k + row * DK, *zv = z + row * DK, *vv = v + row * DV;
            double *a = tok + (size_t)t * (3 * DK + DV), *sg = a + DK, *xs = sg + DK, *uu = xs + DK;
            const double *Sp = St + (size_t)t * SS;
            double *Sn = St + (size_t)(t + 1) * SS;
            for (long c = 0; c < DK; ++c) {
                xs[c] = eA * (double)zv[c];
                sg[c] = logistic(xs[c]);
                a[c] = exp(g_min * sg[c]);
                for (long j = 0; j < DV; ++j)
                    Sn[c * DV + j] = a[c] * Sp[c * DV + j];
            }
            for (long j = 0; j < DV; ++j) {
                double p = 0.0;
                for (long c = 0; c < DK; ++c)
                    p += (double)kv[c] * Sn[c * DV + j];
                uu[j] = (double)vv[j] - p;
            }
            for (long c = 0; c < DK; ++c)
                for (long j = 0; j < DV; ++j)
                    Sn[c * DV + j] += (double)kv[c] * (double)beta[row] * uu[j];
        }
        /* reverse sweep */
        for (size_t e = 0; e < SS; ++e)
            dS[e] = dST ? (double)dST[sbase + e] : 0.0;
        for (long t = T - 1; t >= 0; --t) {
            const size_t row = ((size_t)b * T + t) * H + h;
            const float *qv = q + row * DK, *kv = k + row * DK, *dov = dO + row * DV;
            const double bt = beta[row];
            const double *a = tok + (size_t)t * (3 * DK + DV), *sg = a + DK, *xs = sg + DK, *uu = xs + DK;
            const double *Sprev = St + (size_t)t * SS, *Scur = St + (size_t)(t + 1) * SS;
            /* o = S_t^T q */
            for (long c = 0; c < DK; ++c) {
                double acc = 0.0;
                for (long j = 0; j < DV; ++j) {
                    dS[c * DV + j] += (double)qv[c] * (double)dov[j];
                    acc += Scur[c * DV + j] * (double)dov[j];
                }
                dq[row * DK + c] = acc;
            }
            /* S_t = S' + k e^T, e = beta (v - S'^T k) */
            double db = 0.0;
            for (long j = 0; j < DV; ++j) {
                double acc = 0.0;
                for (long c = 0; c < DK; ++c)
                    acc += (double)kv[c] * dS[c * DV + j];
                de[j] = acc;
                db += acc * uu[j];
                dv[row * DV + j] = bt * acc;
            }
            dbeta[row] = db;
            for (long c = 0; c < DK; ++c) {
                double dkc = 0.0, dac = 0.0;
                for (long j = 0; j < DV; ++j) {
                    const double sprime = a[c] * Sprev[c * DV + j];
                    const double dp = -bt * de[j];
                    dkc += dS[c * DV + j] * bt * uu[j] + sprime * dp;
                    dSp[c * DV + j] = dS[c * DV + j] + (double)kv[c] * dp;
                    dac += dSp[c * DV + j] * Sprev[c * DV + j];
                }
                dk[row * DK + c] = dkc;
                da[c] = dac;
            }
            /* S' = Diag(a) S_{t-1}, a = exp(g_min Sigmoid(e^A z)) */
            for (long c = 0; c < DK; ++c) {
                const double dg = da[c] * a[c];
                const double dx = dg * g_min * sg[c] * (1.0 - sg[c]);
                dz[row * DK + c] = dx * eA;
                dA_unit[u] += dx * xs[c];
                for (long j = 0; j < DV; ++j)
                    dS[c * DV + j] = a[c] * dSp[c * DV + j];
            }
        }
        for (size_t e = 0; e < SS; ++e)
            dS0[sbase + e] = dS[e];
        free(St);
        free(tok);
    }
    for (long h = 0; h < H; ++h)
        dA[h] = 0.0;
    for (long u = 0; u < units; ++u)
        dA[u % H] += dA_unit[u];
    free(dA_unit);
    return failed ? 1 : 0;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
