/*
 * gdn_oracle.h -- plain fp64 CPU oracle for the Gated DeltaNet layer recurrence.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load or call this library. The GPU library never links it, and it
 * shares no source, header or table with the GPU library.
 *
 * What it computes. Source: "Optimizing on-device inference for Apple Silicon"
 * (Perplexity, 2026), section "Qwen creates three distinct workload shapes": each
 * Gated DeltaNet layer compresses earlier tokens into a fixed-size recurrent state; a
 * learned gate sets how much of the old state survives and a delta update writes the
 * current token in, so every token depends on the state left by the token before it.
 * The page gives no formula. The one used here (the gated delta rule) is, per head:
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t * khat_t * khat_t^T) + beta_t * v_t * khat_t^T
 *     o_t = S_t * qhat_t
 *
 * S_t is d_v x d_k. qhat, khat are q and k divided by sqrt(sum of squares + l2_eps), per
 * token and per QK head. V head h reads QK head h / (h_v / h_qk). The output uses the
 * state after the token's own update.
 *
 * Layouts (row-major, C order):
 *   q, k      [n][t][h_qk][d_k]
 *   v         [n][t][h_v][d_v]
 *   g, beta   [n][t][h_v]
 *   state     [n][h_v][d_k][d_v]   element [i][j] holds S[j][i] (the state is stored
 *                                  transposed, d_k-major, as the GPU library stores it)
 *   out       [n][t][h_v][d_v]
 *
 * Every input is fp64. Callers upcast bf16/fp32 data exactly before the call.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Run the recurrence over t tokens for the selected heads.
 *
 *   s0        initial state, or NULL for all zeros.
 *   heads     optional list of flattened head ids (seq * h_v + v_head) to compute;
 *             NULL with n_heads = 0 means every head. Rows of out and s_out for heads
 *             not selected are left untouched.
 *   n_threads worker threads (<= 0: one). Rows of S evolve independently, so the
 *             result is bitwise the same for any thread count.
 *
 * Returns 0 on success, -1 on a bad argument (null pointer, non-positive size,
 * h_v not a multiple of h_qk, head id out of range), -2 if a thread cannot start.
 */
int gdn_oracle_run(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d_k,
                   int32_t d_v, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, const double* s0, double l2_eps,
                   double* out, double* s_out, const int64_t* heads, int64_t n_heads,
                   int32_t n_threads);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
