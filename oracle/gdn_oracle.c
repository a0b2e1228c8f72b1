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

/*
 * Reverse mode of the same recurrence: the gradients of a scalar loss
 *
 *     L = sum(do * o) + sum(dht * ht)
 *
 * with respect to q, k, v, g, beta and h0.  The pages name the backward as
 * the follow-on call and give no formulas for it; these are the chain rule
 * applied to the four lines at the top of this file, token by token in
 * reverse, with P = a_t M_{t-1} (the decayed state) and y = P^T k_t:
 *
 *     dM     += scale q_t do_t^T          dq_t += scale M_t do_t
 *     ddelta  = dM^T k_t                  dk_t += dM delta
 *     dv_t    = b_t ddelta                db_t  = ddelta . (v_t - y)
 *     dy      = -b_t ddelta               dk_t += P dy
 *     dP      = dM + k_t dy^T
 *     dM      = a_t dP                    dg_t  = a_t <dP, M_{t-1}>
 *
 * where dM starts as dht at the end of the sequence, and dh0 is dM once the
 * first token has been undone.  The states before each token are recomputed
 * forward from checkpoints taken every ORACLE_SEG tokens.  A unit is one
 * (sequence, value head) with all value columns, so every sum over columns
 * is formed in one place; dq and dk of a q/k head shared by G value heads
 * are the sum of the G heads' parts, added in head order.
 */
#define ORACLE_SEG 64

typedef struct {
    int64_t B, T;
    int32_t Hqk, Hv, dk, dv;
    const float *q, *k, *v, *g, *beta, *dout;
    double scale;
    const double *h0, *dht;
    const int64_t *cu;
    int64_t N;
    double *dqv, *dkv;     /* [B, T, Hv, dk]: per value head, summed over the group later */
    double *dv_, *dg, *db; /* [B, T, Hv, dv], [B, T, Hv], [B, T, Hv] */
    double *dh0;           /* [N, Hv, dk, dv] or NULL */
    int64_t n_units;
    int64_t next_unit;
} oracle_bwd_problem;

typedef struct {
    double *ck;    /* checkpoints: state before token p0 + s * SEG, s = 0 .. nseg - 1 */
    double *seg;   /* SEG + 1 states of the segment being undone */
    double *dM, *dP, *y, *delta, *dd;
    int64_t ck_cap;
} bwd_buffers;

/* One forward token step on a full dk x dv state (the rule at the top). */
static void fwd_step(const oracle_bwd_problem *P, const double *Min, double *Mout, int64_t p,
                     int32_t j, int32_t hk)
{
    const int32_t dk = P->dk, dv = P->dv;
    const float *kt = P->k + (p * P->Hqk + hk) * dk;
    const float *vt = P->v + (p * P->Hv + j) * dv;
    const int64_t row = p * P->Hv + j;
    const double a = exp((double)P->g[row]);
    const double b = (double)P->beta[row];
    for (int32_t c = 0; c < dv; ++c) {
        double y = 0.0;
        for (int32_t i = 0; i < dk; ++i)
            y += Min[(int64_t)i * dv + c] * (double)kt[i];
        const double delta = b * ((double)vt[c] - a * y);
        for (int32_t i = 0; i < dk; ++i)
            Mout[(int64_t)i * dv + c] = a * Min[(int64_t)i * dv + c] + (double)kt[i] * delta;
    }
}

static int run_bwd_unit(const oracle_bwd_problem *P, int64_t n, int32_t j, bwd_buffers *W)
{
    const int32_t dk = P->dk, dv = P->dv;
    const int64_t S = (int64_t)dk * dv;
    const int32_t hk = j / (P->Hv / P->Hqk);  /* the q/k head of value head j */
    int64_t p0, p1;
    if (P->cu) {
        const int64_t *cn = P->cu + n;
        p0 = cn[0];
        p1 = cn[1];
    } else {
        p0 = n * P->T;
        p1 = p0 + P->T;
    }
    const int64_t len = p1 - p0;
    const int64_t nseg = (len + ORACLE_SEG - 1) / ORACLE_SEG;
    if (nseg > W->ck_cap) {
        double *ck = (double *)realloc(W->ck, sizeof(double) * (size_t)(nseg * S));
        if (!ck)
            return -1;
        W->ck = ck;
        W->ck_cap = nseg;
    }

    /* Forward: the checkpoints. */
    double *M = W->seg, *Mn = W->seg + S;
    const double *h0nj = P->h0 ? P->h0 + ((int64_t)n * P->Hv + j) * S : NULL;
    for (int64_t e = 0; e < S; ++e)
        M[e] = h0nj ? h0nj[e] : 0.0;
    for (int64_t s = 0; s < nseg; ++s) {
        memcpy(W->ck + s * S, M, sizeof(double) * (size_t)S);
        const int64_t e1 = p0 + (s + 1) * ORACLE_SEG < p1 ? p0 + (s + 1) * ORACLE_SEG : p1;
        for (int64_t p = p0 + s * ORACLE_SEG; p < e1; ++p) {
            fwd_step(P, M, Mn, p, j, hk);
            double *t = M;
            M = Mn;
            Mn = t;
        }
    }

    /* Reverse. */
    double *dM = W->dM, *dP = W->dP;
    for (int64_t e = 0; e < S; ++e)
        dM[e] = P->dht ? P->dht[((int64_t)n * P->Hv + j) * S + e] : 0.0;
    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t s0 = p0 + s * ORACLE_SEG;
        const int64_t e1 = s0 + ORACLE_SEG < p1 ? s0 + ORACLE_SEG : p1;
        memcpy(W->seg, W->ck + s * S, sizeof(double) * (size_t)S);
        for (int64_t p = s0; p < e1; ++p)
            fwd_step(P, W->seg + (p - s0) * S, W->seg + (p - s0 + 1) * S, p, j, hk);
        for (int64_t p = e1 - 1; p >= s0; --p) {
            const double *Mprev = W->seg + (p - s0) * S;   /* M_{t-1} */
            const double *Mt = W->seg + (p - s0 + 1) * S;  /* M_t */
            const float *qt = P->q + (p * P->Hqk + hk) * dk;
            const float *kt = P->k + (p * P->Hqk + hk) * dk;
            const float *vt = P->v + (p * P->Hv + j) * dv;
            const float *dot = P->dout + (p * P->Hv + j) * dv;
            const int64_t row = p * P->Hv + j;
            const double a = exp((double)P->g[row]);
            const double b = (double)P->beta[row];
            double *dq = P->dqv + (p * P->Hv + j) * dk;
            double *dkk = P->dkv + (p * P->Hv + j) * dk;
            double *dvv = P->dv_ + (p * P->Hv + j) * dv;

            /* o_t = scale M_t^T q_t */
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int32_t c = 0; c < dv; ++c) {
                    dM[(int64_t)i * dv + c] += P->scale * (double)qt[i] * (double)dot[c];
                    acc += Mt[(int64_t)i * dv + c] * (double)dot[c];
                }
                dq[i] = P->scale * acc;
            }
            /* y = (a M_{t-1})^T k_t, delta = b (v - y) */
            for (int32_t c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    acc += a * Mprev[(int64_t)i * dv + c] * (double)kt[i];
                W->y[c] = acc;
                W->delta[c] = b * ((double)vt[c] - acc);
            }
            /* M_t = P + k_t delta^T */
            double dbeta = 0.0;
            for (int32_t c = 0; c < dv; ++c) {
                double dd = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    dd += dM[(int64_t)i * dv + c] * (double)kt[i];
                W->dd[c] = dd;
                dvv[c] = b * dd;
                dbeta += dd * ((double)vt[c] - W->y[c]);
            }
            P->db[row] = dbeta;
            for (int32_t i = 0; i < dk; ++i) {
                double acc = 0.0, acc2 = 0.0;
                for (int32_t c = 0; c < dv; ++c) {
                    acc += dM[(int64_t)i * dv + c] * W->delta[c];
                    acc2 += a * Mprev[(int64_t)i * dv + c] * (-b * W->dd[c]);
                }
                dkk[i] = acc + acc2;
            }
            /* dP = dM + k dy^T; dM_{t-1} = a dP; dg = a <dP, M_{t-1}> */
            double dga = 0.0;
            for (int32_t i = 0; i < dk; ++i)
                for (int32_t c = 0; c < dv; ++c) {
                    const double v_ = dM[(int64_t)i * dv + c] + (double)kt[i] * (-b * W->dd[c]);
                    dP[(int64_t)i * dv + c] = v_;
                    dga += v_ * Mprev[(int64_t)i * dv + c];
                }
            P->dg[row] = a * dga;
            for (int64_t e = 0; e < S; ++e)
                dM[e] = a * dP[e];
        }
    }
    if (P->dh0)
        memcpy(P->dh0 + ((int64_t)n * P->Hv + j) * S, dM, sizeof(double) * (size_t)S);
    return 0;
}

static void *bwd_worker(void *arg)
{
    oracle_bwd_problem *P = (oracle_bwd_problem *)arg;
    const int64_t S = (int64_t)P->dk * P->dv;
    bwd_buffers W;
    memset(&W, 0, sizeof(W));
    W.seg = (double *)malloc(sizeof(double) * (size_t)((ORACLE_SEG + 1) * S));
    W.dM = (double *)malloc(sizeof(double) * (size_t)S);
    W.dP = (double *)malloc(sizeof(double) * (size_t)S);
    W.y = (double *)malloc(sizeof(double) * (size_t)P->dv);
    W.delta = (double *)malloc(sizeof(double) * (size_t)P->dv);
    W.dd = (double *)malloc(sizeof(double) * (size_t)P->dv);
    void *ret = NULL;
    if (!W.seg || !W.dM || !W.dP || !W.y || !W.delta || !W.dd) {
        ret = (void *)1;
    } else {
        for (;;) {
            const int64_t u = __atomic_fetch_add(&P->next_unit, 1, __ATOMIC_RELAXED);
            if (u >= P->n_units)
                break;
            if (run_bwd_unit(P, u / P->Hv, (int32_t)(u % P->Hv), &W) != 0) {
                ret = (void *)1;
                break;
            }
        }
    }
    free(W.ck); free(W.seg); free(W.dM); free(W.dP); free(W.y); free(W.delta); free(W.dd);
    return ret;
}

/*
 * Returns 0 on success, -1 on a bad argument, -2 on a failed thread start or
 * allocation.  Inputs as for gdn_oracle_fwd, plus dout [B, T, Hv, dv] fp32 and
 * dht [N, Hv, dk, dv] fp64 or NULL (no loss on the final state).  Outputs, all
 * fp64 and zero-filled by the caller: dq, dk [B, T, Hqk, dk]; dv [B, T, Hv, dv];
 * dg, dbeta [B, T, Hv]; dh0 [N, Hv, dk, dv] or NULL.
 */
int gdn_oracle_bwd(int64_t B, int64_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                   const float *q, const float *k, const float *v, const float *g,
                   const float *beta, const float *dout, double scale, const double *h0,
                   const double *dht, const int64_t *cu, int64_t N, double *dq, double *dk_,
                   double *dv_, double *dg, double *dbeta, double *dh0, int32_t nthreads)
{
    if (B < 1 || T < 0 || Hqk < 1 || Hv < 1 || dk < 1 || dv < 1 || Hv % Hqk != 0)
        return -1;
    if (!q || !k || !v || !g || !beta || !dout || !dq || !dk_ || !dv_ || !dg || !dbeta)
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
    const int64_t rows = B * T * (int64_t)Hv;
    double *dqv = (double *)calloc((size_t)(rows * dk), sizeof(double));
    double *dkv = (double *)calloc((size_t)(rows * dk), sizeof(double));
    if (!dqv || !dkv) {
        free(dqv);
        free(dkv);
        return -2;
    }

    oracle_bwd_problem P;
    memset(&P, 0, sizeof(P));
    P.B = B; P.T = T; P.Hqk = Hqk; P.Hv = Hv; P.dk = dk; P.dv = dv;
    P.q = q; P.k = k; P.v = v; P.g = g; P.beta = beta; P.dout = dout;
    P.scale = scale; P.h0 = h0; P.dht = dht; P.cu = cu; P.N = N;
    P.dqv = dqv; P.dkv = dkv; P.dv_ = dv_; P.dg = dg; P.db = dbeta; P.dh0 = dh0;
    P.n_units = N * Hv;
    P.next_unit = 0;

    if (nthreads < 1)
        nthreads = 1;
    if ((int64_t)nthreads > P.n_units)
        nthreads = (int32_t)(P.n_units > 0 ? P.n_units : 1);
    pthread_t *tids = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int rc = 0;
    if (!tids) {
        rc = -2;
    } else {
        int started = 0;
        void *res = NULL;
        for (int i = 0; i < nthreads; ++i) {
            if (pthread_create(&tids[i], NULL, bwd_worker, &P) != 0)
                break;
            ++started;
        }
        for (int i = 0; i < started; ++i) {
            pthread_join(tids[i], &res);
            if (res)
                rc = -2;
        }
        free(tids);
        if (P.next_unit < P.n_units)
            rc = -2;
    }
    if (rc == 0) {
        /* dq, dk of q/k head hk: the sum over its G value heads, in head order. */
        const int32_t G = Hv / Hqk;
        for (int64_t bt = 0; bt < B * T; ++bt)
            for (int32_t hk = 0; hk < Hqk; ++hk)
                for (int32_t i = 0; i < dk; ++i) {
                    double sq = 0.0, sk = 0.0;
                    for (int32_t gi = 0; gi < G; ++gi) {
                        const int64_t r = (bt * Hv + (int64_t)hk * G + gi) * dk + i;
                        sq += dqv[r];
                        sk += dkv[r];
                    }
                    dq[(bt * Hqk + hk) * dk + i] = sq;
                    dk_[(bt * Hqk + hk) * dk + i] = sk;
                }
    }
    free(dqv);
    free(dkv);
    return rc;
}
