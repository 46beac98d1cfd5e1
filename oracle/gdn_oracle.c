/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet layer recurrence.
 *
 * TEST INFRASTRUCTURE: see gdn_oracle.h for who may use it, the definition it follows and
 * the layouts. It is deliberately slow and literal:
 *
 *  - Source for the recurrence: "Optimizing on-device inference for Apple Silicon",
 *    section "Qwen creates three distinct workload shapes" (gate keeps part of the old
 *    state, delta update writes the token in, tokens are processed strictly in order).
 *  - Source for the precision: same page, section "Keep the recurrent state on-chip"
 *    (state and gate in 32-bit floats because rounding compounds over the updates). The
 *    oracle goes further and runs everything in fp64.
 *  - Tokens are processed one after another, exactly as the recurrence is written. The
 *    only rewriting is the distributive law: S (I - beta k k^T) is evaluated as
 *    S - beta (S k) k^T, which is the same matrix with O(d^2) instead of O(d^3) work.
 *  - Rows of S (one per value channel j) never mix: row j of S_t depends only on row j of
 *    S_{t-1}, on v_t[j] and on the shared q, k, g, beta. Threads therefore take disjoint
 *    blocks of rows; no thread ever reads another thread's numbers, so the result does not
 *    depend on the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off (no fast-math), so every product and sum is one
 * IEEE fp64 operation in the order written.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>

#define ROWS_PER_ITEM 16

typedef struct {
    int64_t n, t;
    int32_t h_qk, h_v, d_k, d_v;
    const double *q, *k, *v, *g, *beta, *s0;
    double l2_eps;
    double *out, *s_out;
    const int64_t* heads; /* NULL: every head */
    int64_t n_heads;      /* number of selected heads */
    int64_t row_blocks;   /* blocks of ROWS_PER_ITEM rows per head */
    int64_t n_items;
    int64_t next_item;    /* shared work counter */
    int failed;
} job_t;

/* qhat = x / sqrt(sum_i x_i^2 + eps): the per-head L2 normalisation of q and k. */
static void l2_normalise(const double* x, int32_t d, double eps, double* xhat)
{
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) ss += x[i] * x[i];
    const double norm = sqrt(ss + eps);
    for (int32_t i = 0; i < d; ++i) xhat[i] = x[i] / norm;
}

/* Run rows [row_lo, row_hi) of S for one head over all tokens. */
static int run_item(const job_t* J, int64_t head_id, int32_t row_lo, int32_t row_hi)
{
    const int64_t seq = head_id / J->h_v;
    const int32_t hv = (int32_t)(head_id % J->h_v);
    const int32_t hq = hv / (J->h_v / J->h_qk); /* QK head shared by consecutive V heads */
    const int32_t dk = J->d_k, dv = J->d_v, rows = row_hi - row_lo;

    double* S = (double*)malloc(sizeof(double) * (size_t)rows * (size_t)dk); /* S[j][i] */
    double* qh = (double*)malloc(sizeof(double) * (size_t)dk);
    double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!S || !qh || !kh) {
        free(S); free(qh); free(kh);
        return -1;
    }

    /* S_0: the stored state is d_k-major, element [i][j] = S[j][i]. */
    const int64_t state_base = (seq * J->h_v + hv) * (int64_t)dk * dv;
    for (int32_t r = 0; r < rows; ++r)
        for (int32_t i = 0; i < dk; ++i)
            S[(size_t)r * dk + i] = J->s0 ? J->s0[state_base + (int64_t)i * dv + row_lo + r] : 0.0;

    for (int64_t tt = 0; tt < J->t; ++tt) {
        const int64_t tok = seq * J->t + tt;
        l2_normalise(J->q + (tok * J->h_qk + hq) * dk, dk, J->l2_eps, qh);
        l2_normalise(J->k + (tok * J->h_qk + hq) * dk, dk, J->l2_eps, kh);
        const double alpha = exp(J->g[tok * J->h_v + hv]);
        const double b = J->beta[tok * J->h_v + hv];
        const double* vt = J->v + (tok * J->h_v + hv) * dv;
        double* ot = J->out + (tok * J->h_v + hv) * dv;

        for (int32_t r = 0; r < rows; ++r) {
            double* Sj = S + (size_t)r * dk;
            const double vj = vt[row_lo + r];
            /* u = (S_{t-1} khat)_j */
            double u = 0.0;
            for (int32_t i = 0; i < dk; ++i) u += Sj[i] * kh[i];
            /* S_t[j][i] = alpha * (S_{t-1} (I - beta khat khat^T))[j][i] + beta v_j khat_i */
            for (int32_t i = 0; i < dk; ++i)
                Sj[i] = alpha * (Sj[i] - b * u * kh[i]) + b * vj * kh[i];
            /* o_t[j] = (S_t qhat)_j */
            double o = 0.0;
            for (int32_t i = 0; i < dk; ++i) o += Sj[i] * qh[i];
            ot[row_lo + r] = o;
        }
    }

    for (int32_t r = 0; r < rows; ++r)
        for (int32_t i = 0; i < dk; ++i)
            J->s_out[state_base + (int64_t)i * dv + row_lo + r] = S[(size_t)r * dk + i];

    free(S); free(qh); free(kh);
    return 0;
}

static void* worker(void* arg)
{
    job_t* J = (job_t*)arg;
    for (;;) {
        const int64_t item = __atomic_fetch_add(&J->next_item, 1, __ATOMIC_RELAXED);
        if (item >= J->n_items) break;
        const int64_t sel = item / J->row_blocks;
        const int64_t head_id = J->heads ? J->heads[sel] : sel;
        const int32_t row_lo = (int32_t)(item % J->row_blocks) * ROWS_PER_ITEM;
        int32_t row_hi = row_lo + ROWS_PER_ITEM;
        if (row_hi > J->d_v) row_hi = J->d_v;
        if (run_item(J, head_id, row_lo, row_hi) != 0)
            __atomic_store_n(&J->failed, 1, __ATOMIC_RELAXED);
    }
    return NULL;
}

int gdn_oracle_run(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d_k,
                   int32_t d_v, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, const double* s0, double l2_eps,
                   double* out, double* s_out, const int64_t* heads, int64_t n_heads,
                   int32_t n_threads)
{
    if (n <= 0 || t < 0 || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0) return -1;
    if (h_v % h_qk != 0) return -1;
    if (!s_out || (t > 0 && (!q || !k || !v || !g || !beta || !out))) return -1;
    if (heads) {
        if (n_heads <= 0) return -1;
        for (int64_t i = 0; i < n_heads; ++i)
            if (heads[i] < 0 || heads[i] >= n * h_v) return -1;
    } else {
        n_heads = n * h_v;
    }

    job_t J;
    J.n = n; J.t = t; J.h_qk = h_qk; J.h_v = h_v; J.d_k = d_k; J.d_v = d_v;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s0 = s0; J.l2_eps = l2_eps;
    J.out = out; J.s_out = s_out; J.heads = heads; J.n_heads = n_heads;
    J.row_blocks = (d_v + ROWS_PER_ITEM - 1) / ROWS_PER_ITEM;
    J.n_items = n_heads * J.row_blocks;
    J.next_item = 0;
    J.failed = 0;

    if (n_threads < 1) n_threads = 1;
    if (n_threads > J.n_items) n_threads = (int32_t)J.n_items;
    pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!tids) return -2;
    int32_t started = 0;
    for (; started < n_threads - 1; ++started)
        if (pthread_create(&tids[started], NULL, worker, &J) != 0) break;
    worker(&J); /* the calling thread works too */
    for (int32_t i = 0; i < started; ++i) pthread_join(tids[i], NULL);
    free(tids);
    return J.failed ? -2 : 0;
}
