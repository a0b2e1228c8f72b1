/*
 * gdn_oracle.c -- the fp64 token-by-token gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the CPU oracle that the HIP library
 * is checked against.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the library never does, and the
 * two share no code.
 *
 * What it computes (the recurrence the pages state in closed form for the
 * Gated DeltaNet token mixer, and the reference-implementation role the
 * jax-linear-attention page gives its "token-by-token reference" in
 * "How it works"):
 *
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
 *
 * with a_t = exp(g_t) (g is the natural-log decay, jax-linear-attention page,
 * "Quick start") and b_t the write strength beta.  The state here is stored
 * transposed, M = S^T, a dk x dv matrix whose element (i, c) couples key
 * dimension i to value dimension c (the (B, H, K, V) state of the same
 * "Quick start").  Transposing the formula gives, per token:
 *
 *     y     = M^T k_t                     (the prediction before the decay)
 *     delta = b_t (v_t - a_t y)
 *     M     = a_t M + k_t delta^T
 *     o_t   = scale * M^T q_t             (after the write: o_t sees token t)
 *
 * Every sequence starts from its initial state (or zero) and runs its own
 * tokens only: with cu_seqlens, sequence n is tokens [cu[n], cu[n+1]) of the
 * single packed row, which is the per-document reset of "How it works" on the
 * jax-linear-attention page.  Without cu_seqlens, sequence n is batch row n.
 *
 * All arithmetic is IEEE fp64 with no contraction (built with
 * -ffp-contract=off).  Inputs arrive as fp32, which holds bf16 and fp32 input
 * values exactly.  Work is split over independent (sequence, value head,
 * value-column block) units: value columns of M evolve independently, so the
 * split never divides a reduction and the result does not depend on the
 * thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_COL_BLOCK 32

typedef struct {
    int64_t B, T;
    int32_t Hqk, Hv, dk, dv;
    const float *q, *k, *v, *g, *beta;
    double scale;
    const double *h0;      /* [N, Hv, dk, dv] or NULL (zero state) */
    const int64_t *cu;     /* [N + 1] token offsets into the one packed row, or NULL */
    int64_t N;             /* number of sequences */
    double *o;             /* [B, T, Hv, dv] */
    double *ht;            /* [N, Hv, dk, dv] or NULL */
    int64_t n_units;
    int32_t n_col_blocks;
    int64_t next_unit;     /* shared work counter */
} oracle_problem;

/* One unit: sequence n, value head j, value columns [c0, c1). */
static void run_unit(const oracle_problem *P, int64_t n, int32_t j, int32_t c0, int32_t c1,
                     double *M, double *delta)
{
    const int32_t dk = P->dk, dv = P->dv;
    const int32_t G = P->Hv / P->Hqk;
    const int32_t hk = j / G; /* the q/k head this value head reads */
    const int32_t w = c1 - c0;
    int64_t p0, p1;
    if (P->cu) {
        p0 = P->cu[n];
        p1 = P->cu[n + 1];
    } else {
        p0 = n * P->T;
        p1 = p0 + P->T;
    }

    for (int32_t i = 0; i < dk; ++i)
        for (int32_t c = 0; c < w; ++c)
            M[(int64_t)i * w + c] =
                P->h0 ? P->h0[(((int64_t)n * P->Hv + j) * dk + i) * dv + c0 + c] : 0.0;

    for (int64_t p = p0; p < p1; ++p) {
        const float *kt = P->k + (p * P->Hqk + hk) * dk;
        const float *qt = P->q + (p * P->Hqk + hk) * dk;
        const float *vt = P->v + (p * P->Hv + j) * dv + c0;
        const double a = exp((double)P->g[p * P->Hv + j]);
        const double b = (double)P->beta[p * P->Hv + j];

        for (int32_t c = 0; c < w; ++c) {
            double y = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                y += M[(int64_t)i * w + c] * (double)kt[i];
            delta[c] = b * ((double)vt[c] - a * y);
        }
        for (int32_t i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            for (int32_t c = 0; c < w; ++c)
                M[(int64_t)i * w + c] = a * M[(int64_t)i * w + c] + ki * delta[c];
        }
        double *ot = P->o + (p * P->Hv + j) * dv + c0;
        for (int32_t c = 0; c < w; ++c) {
            double acc = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                acc += M[(int64_t)i * w + c] * (double)qt[i];
            ot[c] = P->scale * acc;
        }
    }

    if (P->ht)
        for (int32_t i = 0; i < dk; ++i)
            for (int32_t c = 0; c < w; ++c)
                P->ht[(((int64_t)n * P->Hv + j) * dk + i) * dv + c0 + c] = M[(int64_t)i * w + c];
}

static void *worker(void *arg)
{
    oracle_problem *P = (oracle_problem *)arg;
    double *M = (double *)malloc(sizeof(double) * (size_t)P->dk * ORACLE_COL_BLOCK);
    double *delta = (double *)malloc(sizeof(double) * ORACLE_COL_BLOCK);
    if (!M || !delta) {
        free(M);
        free(delta);
        return (void *)1;
    }
    for (;;) {
        const int64_t u = __atomic_fetch_add(&P->next_unit, 1, __ATOMIC_RELAXED);
        if (u >= P->n_units)
            break;
        const int32_t cb = (int32_t)(u % P->n_col_blocks);
        const int64_t nj = u / P->n_col_blocks;
        const int32_t j = (int32_t)(nj % P->Hv);
        const int64_t n = nj / P->Hv;
        const int32_t c0 = cb * ORACLE_COL_BLOCK;
        const int32_t c1 = c0 + ORACLE_COL_BLOCK < P->dv ? c0 + ORACLE_COL_BLOCK : P->dv;
        run_unit(P, n, j, c0, c1, M, delta);
    }
    free(M);
    free(delta);
    return NULL;
}

/*
 * Returns 0 on success, -1 on a bad argument, -2 if a thread could not be
 * started or a work buffer could not be allocated.
 *
 * q, k: [B, T, Hqk, dk]; v: [B, T, Hv, dv]; g, beta: [B, T, Hv]; all fp32,
 * contiguous.  With cu (int64 [N + 1]) B must be 1, cu[0] = 0, cu
 * non-decreasing and cu[N] = T.  o: [B, T, Hv, dv] fp64; ht: [N, Hv, dk, dv]
 * fp64 or NULL.  Tokens outside every sequence (none, when cu is valid) are
 * left untouched in o.
 */
int gdn_oracle_fwd(int64_t B, int64_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                   const float *q, const float *k, const float *v, const float *g,
                   const float *beta, double scale, const double *h0, const int64_t *cu,
                   int64_t N, double *o, double *ht, int32_t nthreads)
{
    if (B < 1 || T < 0 || Hqk < 1 || Hv < 1 || dk < 1 || dv < 1 || Hv % Hqk != 0)
        return -1;
    if (!q || !k || !v || !g || !beta || !o)
        return -1;
    if (cu) {
        if (B != 1 || N < 1 || cu[0] != 0 || cu[N] != T)
            return -1;
        for (int64_t n = 0; n < N; ++n)
            if (cu[n + 1] < cu[n])
                return -1;
    } else {
        N = B;
    }

    oracle_problem P;
    memset(&P, 0, sizeof(P));
    P.B = B; P.T = T; P.Hqk = Hqk; P.Hv = Hv; P.dk = dk; P.dv = dv;
    P.q = q; P.k = k; P.v = v; P.g = g; P.beta = beta;
    P.scale = scale; P.h0 = h0; P.cu = cu; P.N = N; P.o = o; P.ht = ht;
    P.n_col_blocks = (dv + ORACLE_COL_BLOCK - 1) / ORACLE_COL_BLOCK;
    P.n_units = N * Hv * P.n_col_blocks;
    P.next_unit = 0;

    if (nthreads < 1)
        nthreads = 1;
    if ((int64_t)nthreads > P.n_units)
        nthreads = (int32_t)(P.n_units > 0 ? P.n_units : 1);

    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tids)
        return -2;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tids[i], NULL, worker, &P) != 0)
            break;
        ++started;
    }
    for (int i = 0; i < started; ++i)
        pthread_join(tids[i], NULL);
    free(tids);
    /* A worker claims units only after its buffers exist, and every running
       worker drains the queue, so the result is complete exactly when every
       unit has been claimed. */
    return P.next_unit >= P.n_units ? 0 : -2;
}
