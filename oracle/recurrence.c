/*
 * Float64 CPU oracle for the decode-time recurrences of gated delta-rule
 * linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the GPU library and must never be used as a
 * fallback for it.
 *
 * What it computes (per state, i.e. per (sequence, layer, head), one step at
 * a time, in the order the formulas are written):
 *
 *   Gated DeltaNet  S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   KDA             S_t = S_{t-1} diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   RWKV6-style     S_t = S_{t-1} diag(w_t) + v_t k_t^T
 *   gated (GDN-2)   S_t = S_{t-1} diag(alpha_t) (I - (e_t * k_t) k_t^T) + (w_t * v_t) k_t^T
 *   readout         o_t = S_t q_t
 *
 * with S a d_v x d_k matrix (row = value channel, column = key channel),
 * alpha_t = exp(g_t) from the stored log-decay g_t.  The DeltaLog page
 * ("DeltaLog: Deferred Materialization of Recurrent States for Linear
 * Attention Decoding", Technical Summary, Kernel Implementation) names the
 * three operators and their decay granularity: a head-wise scalar decay with
 * the delta-rule correction (GDN), a per-key decay with the correction (KDA),
 * and a per-key decay with raw-value updates (RWKV6).  The Gated DeltaNet-2
 * abstract on the CARVE page ("Explore similar work") fixes how they nest:
 * KDA becomes Gated DeltaNet when its decay collapses to one scalar.  The
 * deferred (base + log) schedule changes none of this arithmetic (DeltaLog
 * page, Methodology), so the oracle is the plain recurrence.
 *
 * The gated form follows the Gated DeltaNet-2 abstract: KDA's single scalar
 * beta is split into a channel-wise erase gate e_t on the key channels
 * (how much of the stored content along k_t is read out and removed) and a
 * channel-wise write gate w_t on the value channels (how much of v_t is
 * committed), and it becomes KDA when both gates are the same scalar.
 *
 * Every product is written out as the formula's terms: the decayed state,
 * its product with k, the two rank-one terms, then the readout.  Inputs are
 * the exact values the GPU consumes (bf16 or fp32, passed here as float32)
 * and are upcast exactly to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_GDN = 0, ORACLE_KDA = 1, ORACLE_RWKV6 = 2, ORACLE_GDN2 = 3 };

/* S[i][j] *= a  (the scalar head-wise decay) */
static void scale_all(int dv, int dk, double *S, double a)
{
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] *= a;
}

/* S <- S diag(a): column j (key channel j) is scaled by a[j] */
static void scale_columns(int dv, int dk, double *S, const double *a)
{
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] *= a[j];
}

/* y = S x  (y has d_v entries, x has d_k) */
static void matvec(int dv, int dk, const double *S, const double *x, double *y)
{
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j)
            acc += S[(size_t)i * dk + j] * x[j];
        y[i] = acc;
    }
}

/* S <- S + c * a b^T  (a has d_v entries, b has d_k) */
static void add_outer(int dv, int dk, double *S, double c, const double *a, const double *b)
{
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j)
            S[(size_t)i * dk + j] += c * a[i] * b[j];
}

/* One state through steps t_first..T-1. */
static void run_one(int variant, int64_t pair, int64_t n_pairs, int dk, int dv, int T,
                    int t_first, const float *S0, const double *S0d, const float *q,
                    const float *k, const float *v, const float *g, const float *beta,
                    double *o, double *S_out, double *work)
{
    double *S = S_out + (size_t)pair * dv * dk;
    double *qd = work;            /* d_k */
    double *kd = qd + dk;         /* d_k */
    double *vd = kd + dk;         /* d_v */
    double *al = vd + dv;         /* d_k */
    double *Sk = al + dk;         /* d_v */
    double *ot = Sk + dv;         /* d_v */
    double *ek = ot + dv;         /* d_k */
    double *wv = ek + dk;         /* d_v */

    for (size_t e = 0; e < (size_t)dv * dk; ++e)
        S[e] = S0d ? S0d[(size_t)pair * dv * dk + e]
             : S0  ? (double)S0[(size_t)pair * dv * dk + e] : 0.0;

    for (int t = 0; t < T; ++t) {
        double *o_t = o + ((size_t)t * n_pairs + pair) * dv;
        if (t < t_first) {
            for (int i = 0; i < dv; ++i)
                o_t[i] = 0.0;
            continue;
        }
        const size_t row = (size_t)t * n_pairs + pair;
        for (int j = 0; j < dk; ++j) {
            qd[j] = (double)q[row * dk + j];
            kd[j] = (double)k[row * dk + j];
        }
        for (int i = 0; i < dv; ++i)
            vd[i] = (double)v[row * dv + i];

        if (variant == ORACLE_GDN) {
            /* S <- alpha S (I - beta k k^T) + beta v k^T */
            const double alpha = exp((double)g[row]);
            const double b = (double)beta[row];
            scale_all(dv, dk, S, alpha);          /* alpha S            */
            matvec(dv, dk, S, kd, Sk);            /* (alpha S) k        */
            add_outer(dv, dk, S, -b, Sk, kd);     /* - beta (alpha S k) k^T */
            add_outer(dv, dk, S, b, vd, kd);      /* + beta v k^T       */
        } else if (variant == ORACLE_KDA) {
            /* S <- S diag(alpha) (I - beta k k^T) + beta v k^T */
            const double b = (double)beta[row];
            for (int j = 0; j < dk; ++j)
                al[j] = exp((double)g[row * dk + j]);
            scale_columns(dv, dk, S, al);         /* S diag(alpha)      */
            matvec(dv, dk, S, kd, Sk);
            add_outer(dv, dk, S, -b, Sk, kd);
            add_outer(dv, dk, S, b, vd, kd);
        } else if (variant == ORACLE_GDN2) {
            /* S <- S diag(alpha) (I - (e * k) k^T) + (w * v) k^T, with the
             * erase gate e [d_k] and then the write gate w [d_v] in beta */
            const float *gate = beta + row * (size_t)(dk + dv);
            for (int j = 0; j < dk; ++j) {
                al[j] = exp((double)g[row * dk + j]);
                ek[j] = (double)gate[j] * kd[j];
            }
            for (int i = 0; i < dv; ++i)
                wv[i] = (double)gate[dk + i] * vd[i];
            scale_columns(dv, dk, S, al);         /* S diag(alpha)      */
            matvec(dv, dk, S, ek, Sk);            /* S diag(alpha) (e * k) */
            add_outer(dv, dk, S, -1.0, Sk, kd);   /* - (S diag(alpha) (e * k)) k^T */
            add_outer(dv, dk, S, 1.0, wv, kd);    /* + (w * v) k^T      */
        } else {
            /* S <- S diag(w) + v k^T */
            for (int j = 0; j < dk; ++j)
                al[j] = exp((double)g[row * dk + j]);
            scale_columns(dv, dk, S, al);
            add_outer(dv, dk, S, 1.0, vd, kd);
        }
        matvec(dv, dk, S, qd, ot);                /* o_t = S_t q_t      */
        for (int i = 0; i < dv; ++i)
            o_t[i] = ot[i];
    }
}

/*
 * Run the recurrence for n_pairs independent states over T steps.
 *
 *   S0      [n_pairs, d_v, d_k] float32, or NULL for zero initial states
 *   q, k    [T, n_pairs, d_k]   float32 (exact bf16/fp32 input values)
 *   v       [T, n_pairs, d_v]   float32
 *   g       [T, n_pairs] (GDN) or [T, n_pairs, d_k] (KDA, RWKV6, gated) float32 log-decay
 *   beta    [T, n_pairs] float32; [T, n_pairs, d_k + d_v] for the gated form
 *           (erase gate, then write gate); ignored (may be NULL) for RWKV6
 *   t_start [n_pairs] int32 first step a state takes, or NULL (all start at 0);
 *           outputs before it are 0
 *   o       [T, n_pairs, d_v] float64 out
 *   S_out   [n_pairs, d_v, d_k] float64 out (state after the last step)
 *   n_threads  OpenMP threads (<= 0: library default)
 *
 * Returns 0, or -1 for invalid arguments, -2 if scratch memory is unavailable.
 */
static int run_all(int variant, int64_t n_pairs, int d_k, int d_v, int T, const float *S0,
                   const double *S0d, const float *q, const float *k, const float *v,
                   const float *g, const float *beta, const int32_t *t_start, double *o,
                   double *S_out, int n_threads);

int oracle_run(int variant, int64_t n_pairs, int d_k, int d_v, int T, const float *S0,
               const float *q, const float *k, const float *v, const float *g,
               const float *beta, const int32_t *t_start, double *o, double *S_out,
               int n_threads)
{
    return run_all(variant, n_pairs, d_k, d_v, T, S0, NULL, q, k, v, g, beta, t_start, o,
                   S_out, n_threads);
}

/* The same with a float64 initial state S0d [n_pairs, d_v, d_k] (a state
 * that is not an fp32 value, e.g. a dequantised base). */
int oracle_run_f64_state(int variant, int64_t n_pairs, int d_k, int d_v, int T,
                         const double *S0d, const float *q, const float *k, const float *v,
                         const float *g, const float *beta, const int32_t *t_start, double *o,
                         double *S_out, int n_threads)
{
    if (!S0d)
        return -1;
    return run_all(variant, n_pairs, d_k, d_v, T, NULL, S0d, q, k, v, g, beta, t_start, o,
                   S_out, n_threads);
}

static int run_all(int variant, int64_t n_pairs, int d_k, int d_v, int T, const float *S0,
                   const double *S0d, const float *q, const float *k, const float *v,
                   const float *g, const float *beta, const int32_t *t_start, double *o,
                   double *S_out, int n_threads)
{
    if (variant < ORACLE_GDN || variant > ORACLE_GDN2 || n_pairs < 0 || d_k <= 0 ||
        d_v <= 0 || T < 0 || !q || !k || !v || !g || !o || !S_out)
        return -1;
    if (variant != ORACLE_RWKV6 && !beta)
        return -1;
    const size_t work_len = (size_t)4 * d_k + (size_t)4 * d_v;
    int failed = 0;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double *work = (double *)malloc(work_len * sizeof(double));
        if (!work) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t p = 0; p < n_pairs; ++p) {
            if (!work)
                continue;
            const int t0 = t_start ? t_start[p] : 0;
            run_one(variant, p, n_pairs, d_k, d_v, T, t0, S0, S0d, q, k, v, g, beta, o, S_out,
                    work);
        }
        free(work);
    }
    return failed ? -2 : 0;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
