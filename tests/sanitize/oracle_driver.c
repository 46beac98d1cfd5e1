/* Drives the fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer: several
 * shapes, with and without an initial state, a head subset, one and several threads, and
 * rejected arguments. Exits non-zero on a mismatch between thread counts or an unexpected
 * return code; the sanitizers abort on any invalid access. Inputs are plain pseudo-random
 * numbers (xorshift64), not the library's input recipe. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn_oracle.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uni(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

static double* filled(size_t n, double lo, double hi)
{
    double* p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}

static int run_shape(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d, int with_s0)
{
    const size_t nqk = (size_t)(n * t * h_qk * d), nv = (size_t)(n * t * h_v * d);
    const size_t ngb = (size_t)(n * t * h_v), ns = (size_t)(n * h_v * d * d);
    double *q = filled(nqk, -1, 1), *k = filled(nqk, -1, 1), *v = filled(nv, -1, 1);
    double *g = filled(ngb, -0.5, 0), *b = filled(ngb, 0, 1);
    double* s0 = with_s0 ? filled(ns, -0.05, 0.05) : NULL;
    double *o1 = calloc(nv ? nv : 1, sizeof(double)), *s1 = calloc(ns, sizeof(double));
    double *o3 = calloc(nv ? nv : 1, sizeof(double)), *s3 = calloc(ns, sizeof(double));
    int bad = 0;
    if (gdn_oracle_run(n, t, h_qk, h_v, d, d, q, k, v, g, b, s0, 1e-6, o1, s1, NULL, 0, 1) != 0) bad = 1;
    if (gdn_oracle_run(n, t, h_qk, h_v, d, d, q, k, v, g, b, s0, 1e-6, o3, s3, NULL, 0, 3) != 0) bad = 1;
    if (memcmp(o1, o3, nv * sizeof(double)) || memcmp(s1, s3, ns * sizeof(double))) bad = 1;
    /* a head subset leaves the other heads' rows untouched */
    const int64_t heads[2] = {0, n * h_v - 1};
    double *os = calloc(nv ? nv : 1, sizeof(double)), *ss = calloc(ns, sizeof(double));
    if (gdn_oracle_run(n, t, h_qk, h_v, d, d, q, k, v, g, b, s0, 1e-6, os, ss, heads, 2, 2) != 0) bad = 1;
    free(q); free(k); free(v); free(g); free(b); free(s0);
    free(o1); free(s1); free(o3); free(s3); free(os); free(ss);
    if (bad) fprintf(stderr, "shape n=%lld t=%lld h_qk=%d h_v=%d d=%d s0=%d failed\n",
                     (long long)n, (long long)t, h_qk, h_v, d, with_s0);
    return bad;
}

int main(void)
{
    int bad = 0;
    bad |= run_shape(2, 37, 2, 4, 16, 1);
    bad |= run_shape(1, 1, 1, 2, 32, 0);
    bad |= run_shape(3, 9, 1, 3, 8, 1);
    bad |= run_shape(1, 64, 2, 2, 16, 0);
    double x = 0;
    const int64_t bad_head = 99;
    /* rejected arguments */
    if (gdn_oracle_run(1, 1, 2, 3, 4, 4, &x, &x, &x, &x, &x, NULL, 1e-6, &x, &x, NULL, 0, 1) != -1) bad = 1;
    if (gdn_oracle_run(1, 1, 1, 1, 4, 4, NULL, &x, &x, &x, &x, NULL, 1e-6, &x, &x, NULL, 0, 1) != -1) bad = 1;
    if (gdn_oracle_run(1, 1, 1, 1, 1, 1, &x, &x, &x, &x, &x, NULL, 1e-6, &x, &x, &bad_head, 1, 1) != -1) bad = 1;
    printf("oracle driver %s\n", bad ? "FAILED" : "ok");
    return bad;
}
