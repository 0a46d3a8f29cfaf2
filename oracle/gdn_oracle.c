/*
 * Gated DeltaNet recurrence, fp64, sequential in time.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plainly-written CPU oracle
 * that the GPU library is checked against.  Nothing in the product path may
 * link, load or call it; it shares no source with the GPU library.
 *
 * Source of the arithmetic ("Qwen3.8-27B: from model structure to the vLLM
 * inference dataflow", section 01 LAYER-BY-LAYER, per-layer operator table, GDN
 * row; the same update in section 03 MEMORY LABS, GDN state lab; section 08
 * EVIDENCE MATRIX, row on decay-before-read):
 *
 *   for every token t of a request, per value head h with key head kh:
 *     Sbar = alpha_t * S                      (decay first)
 *     e    = v_t - Sbar k_t                   (error read from the DECAYED state)
 *     S    = Sbar + beta_t * e k_t^T          (rank-1 delta write)
 *     o_t  = S q_t / sqrt(d_k)                (read after the write)
 *
 * S is stored as [d_v][d_k] (row i = value channel, column j = key channel), so
 * "S k" contracts over the key channel.  Value head h reads key head
 * h / (Hv / Hk): contiguous groups, as the page's 4-way tensor-parallel table
 * places key heads 0-3 with value heads 0-11 on one rank.
 *
 * alpha and beta arrive already mapped from the raw projections (the mapping
 * is done in oracle.py in numpy); this file only runs the recurrence.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (request, value head) unit.  S points at that unit's [dv][dk] state. */
static void recur_unit(int64_t t0, int64_t t1, int32_t h, int32_t kh,
                       int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta,
                       double *S, double *o, double *e /* dv scratch */)
{
    const double inv_sqrt_dk = 1.0 / sqrt((double)dk);
    for (int64_t t = t0; t < t1; ++t) {
        const double a = alpha[t * Hv + h];
        const double b = beta[t * Hv + h];
        const double *kt = k + (t * Hk + kh) * dk;
        const double *qt = q + (t * Hk + kh) * dk;
        const double *vt = v + (t * Hv + h) * dv;
        double *ot = o + (t * Hv + h) * dv;

        /* Sbar = alpha * S */
        for (int32_t i = 0; i < dv; ++i)
            for (int32_t j = 0; j < dk; ++j)
                S[i * dk + j] *= a;

        /* e = v - Sbar k */
        for (int32_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < dk; ++j)
                acc += S[i * dk + j] * kt[j];
            e[i] = vt[i] - acc;
        }

        /* S = Sbar + beta e k^T */
        for (int32_t i = 0; i < dv; ++i)
            for (int32_t j = 0; j < dk; ++j)
                S[i * dk + j] += b * e[i] * kt[j];

        /* o = S q / sqrt(dk) */
        for (int32_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < dk; ++j)
                acc += S[i * dk + j] * qt[j];
            ot[i] = acc * inv_sqrt_dk;
        }
    }
}

/*
 * Run the recurrence over a packed batch.
 *   q, k      [T, Hk, dk]
 *   v, o      [T, Hv, dv]
 *   alpha,beta[T, Hv]
 *   qsl       [nreq + 1]   request r owns tokens qsl[r] .. qsl[r+1]-1
 *   slot      [nreq]       state slot of request r (distinct, checked by caller)
 *   has_init  [nreq]       0: the request starts from a zero state
 *   state     [nslots, Hv, dv, dk]  read and written in place
 * Returns 0, or -1 if an internal allocation fails.
 */
int oracle_gdn_recurrence(int32_t nreq, const int32_t *qsl, const int32_t *slot,
                          const uint8_t *has_init, int32_t Hk, int32_t Hv,
                          int32_t dk, int32_t dv, const double *q,
                          const double *k, const double *v,
                          const double *alpha, const double *beta,
                          double *state, double *o)
{
    const int32_t group = Hv / Hk;
    const int64_t units = (int64_t)nreq * Hv;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t u = 0; u < units; ++u) {
        const int32_t r = (int32_t)(u / Hv);
        const int32_t h = (int32_t)(u % Hv);
        const int64_t t0 = qsl[r], t1 = qsl[r + 1];
        if (t1 <= t0)
            continue; /* empty request: its slot is left untouched */
        double *S = state + ((int64_t)slot[r] * Hv + h) * (int64_t)dv * dk;
        if (!has_init[r])
            memset(S, 0, sizeof(double) * (size_t)dv * (size_t)dk);
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!e) {
            failed = 1;
            continue;
        }
        recur_unit(t0, t1, h, h / group, Hk, Hv, dk, dv, q, k, v, alpha, beta,
                   S, o, e);
        free(e);
    }
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following parallel regions (n >= 1; for timing the core
 * on one thread beside all of them). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
