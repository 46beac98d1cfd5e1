"""Independent fp64 chunked (UT/WY) evaluation of the Gated DeltaNet recurrence.

Test-only: it exists to pin the oracle. It shares nothing with the oracle (a plain token
loop in C) and nothing with the GPU library. "Optimizing on-device inference for Apple
Silicon", section "Qwen creates three distinct workload shapes", states that prefill can
either scan the tokens directly or re-block the updates into chunks that expose matrix
work, and that both give the same result; this module is the re-blocked form, derived
here from the recurrence, so agreement with the token-by-token oracle pins both.

Derivation (per head, M = S^T of shape d_k x d_v, tokens r = 1..C of one chunk, M0 the
state entering the chunk, khat/qhat normalised rows):
  gamma_r = g_1 + ... + g_r,  Gamma_r = exp(gamma_r)
  each value column evolves as m_r = alpha_r m_{r-1} + khat_r u_r with
  u_r = beta_r (v_r - alpha_r khat_r . m_{r-1}); unrolling m_{r-1} gives the lower
  triangular system (I + A) U = diag(beta) V - diag(beta Gamma) Khat M0 with
  A[r, s] = beta_r exp(gamma_r - gamma_s) (khat_r . khat_s) for s < r, so
  U = (I + A)^{-1} (diag(beta) V - diag(beta Gamma) Khat M0)
  O = diag(Gamma) Qhat M0 + (L o Qhat Khat^T) U,  L[r, s] = exp(gamma_r - gamma_s), s <= r
  M_C = Gamma_C M0 + Khat^T diag(exp(gamma_C - gamma)) U
"""
import numpy as np


def _normalise(x, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def chunked(q, k, v, g, beta, state_in, chunk, l2_eps=1e-6):
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    n, t, h_qk, d_k = q.shape
    h_v, d_v = v.shape[2], v.shape[3]
    grp = h_v // h_qk
    out = np.zeros((n, t, h_v, d_v))
    s_out = np.zeros((n, h_v, d_k, d_v))
    for b in range(n):
        for h in range(h_v):
            M = (np.zeros((d_k, d_v)) if state_in is None
                 else np.array(state_in[b, h], dtype=np.float64))
            for c0 in range(0, t, chunk):
                c1 = min(t, c0 + chunk)
                K = _normalise(k[b, c0:c1, h // grp], l2_eps)
                Q = _normalise(q[b, c0:c1, h // grp], l2_eps)
                V = v[b, c0:c1, h]
                bt = beta[b, c0:c1, h]
                gam = np.cumsum(g[b, c0:c1, h])
                decay = np.exp(gam[:, None] - gam[None, :])  # exp(gamma_r - gamma_s)
                A = np.tril(bt[:, None] * decay * (K @ K.T), -1)
                Tinv = np.linalg.inv(np.eye(c1 - c0) + A)
                U = Tinv @ (bt[:, None] * V - (bt * np.exp(gam))[:, None] * (K @ M))
                L = np.tril(decay)
                out[b, c0:c1, h] = np.exp(gam)[:, None] * (Q @ M) + (L * (Q @ K.T)) @ U
                M = np.exp(gam[-1]) * M + K.T @ (np.exp(gam[-1] - gam)[:, None] * U)
            s_out[b, h] = M
    return out, s_out
