"""Pins for the fp64 oracle: results fixed by the mathematics of the recurrence.

Each pin takes `run(q, k, v, g, beta, state_in, l2_eps, threads=None)` returning
(out, state_out) in the oracle's layouts, so the same pins also run against deliberately
broken builds of the oracle (test_oracle_mutants.py) to show that they catch mistakes.

The recurrence (gated delta rule; "Optimizing on-device inference for Apple Silicon",
section "Qwen creates three distinct workload shapes", describes it in words):
  S_t = exp(g_t) S_{t-1} (I - beta_t khat_t khat_t^T) + beta_t v_t khat_t^T,  o_t = S_t qhat_t
with S stored transposed (state[i][j] = S[j][i]).

None of the pins re-evaluates the oracle's own token loop: each one checks a closed form,
an invariant, an exact special case, or an independently derived evaluation.
"""
import numpy as np

from chunked_ref import chunked


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def rand_case(seed, n=1, t=24, h_qk=1, h_v=2, d_k=8, d_v=8, s0_scale=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, t, h_qk, d_k))
    k = rng.standard_normal((n, t, h_qk, d_k))
    v = rng.standard_normal((n, t, h_v, d_v))
    g = np.log(_sigmoid(rng.normal(2.0, 1.0, (n, t, h_v))))
    beta = _sigmoid(rng.standard_normal((n, t, h_v)))
    s0 = None if s0_scale == 0 else rng.normal(0.0, s0_scale, (n, h_v, d_k, d_v))
    return q, k, v, g, beta, s0


def _unit(x, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------- pins
def pin_identity(run):
    """beta = 0 and g = 0: every update is the identity, so S_t = S_0 exactly and
    o_t = S_0 qhat_t."""
    q, k, v, g, beta, s0 = rand_case(1, n=2, t=17, h_qk=2, h_v=4, d_k=8, d_v=6)
    g[:] = 0.0
    beta[:] = 0.0
    out, st = run(q, k, v, g, beta, s0, 1e-6)
    assert np.array_equal(st, s0), "state changed although beta = g = 0"
    qh = _unit(q, 1e-6)
    for h in range(4):
        expect = np.einsum("ntd,ndj->ntj", qh[:, :, h // 2], s0[:, h])
        assert _rel(out[:, :, h], expect) < 1e-13


def pin_decay_only(run):
    """beta = 0: S_t = exp(g_1 + ... + g_t) S_0 and o_t = exp(g_1 + ... + g_t) S_0 qhat_t."""
    q, k, v, g, beta, s0 = rand_case(2, t=40, d_k=8, d_v=8)
    beta[:] = 0.0
    out, st = run(q, k, v, g, beta, s0, 1e-6)
    gam = np.cumsum(g, axis=1)  # [n, t, h_v]
    qh = _unit(q, 1e-6)
    for h in range(2):
        assert _rel(st[0, h], np.exp(gam[0, -1, h]) * s0[0, h]) < 1e-12
        expect = np.exp(gam[0, :, h])[:, None] * (qh[0, :, 0] @ s0[0, h])
        assert _rel(out[0, :, h], expect) < 1e-12


def pin_retrieval(run):
    """g = 0, beta = 1 (plain delta rule): after writing (k_t, v_t) the state returns
    v_t for the unit key, S_t khat_t = v_t. With q = k the output is therefore v_t."""
    q, k, v, g, beta, s0 = rand_case(3, n=2, t=30, h_qk=2, h_v=4, d_k=8, d_v=5)
    g[:] = 0.0
    beta[:] = 1.0
    out, st = run(k, k, v, g, beta, s0, 0.0)
    assert np.max(np.abs(out - v)) < 1e-12 * np.max(np.abs(v))
    kh = _unit(k[:, -1], 0.0)  # [n, h_qk, d_k]
    for h in range(4):
        last = np.einsum("ni,nij->nj", kh[:, h // 2], st[:, h])
        assert np.max(np.abs(last - v[:, -1, h])) < 1e-12 * np.max(np.abs(v))


def pin_orthonormal_keys(run):
    """Keys along distinct axes e_c (any positive length): the projections commute and
    the closed form per state column c of S is
      c never written:      S_t[:, c] = exp(sum_{s<=t} g_s) S_0[:, c]
      c written at tau:     S_t[:, c] = exp(sum_{tau<s<=t} g_s) *
                            (exp(g_tau)(1 - beta_tau) exp(sum_{s<tau} g_s) S_0[:, c]
                             + beta_tau v_tau)          for t >= tau."""
    rng = np.random.default_rng(4)
    t, d_k, d_v = 6, 9, 4
    q, k, v, g, beta, s0 = rand_case(4, t=t, h_qk=1, h_v=2, d_k=d_k, d_v=d_v)
    axes = rng.permutation(d_k)[:t]
    k[:] = 0.0
    for s in range(t):
        k[0, s, 0, axes[s]] = rng.uniform(0.5, 3.0)
    out, st = run(q, k, v, g, beta, s0, 0.0)
    qh = _unit(q, 0.0)
    for h in range(2):
        gam = np.concatenate([[0.0], np.cumsum(g[0, :, h])])  # gam[t] = sum_{s<=t}
        S0 = s0[0, h].T  # d_v x d_k
        for tt in range(1, t + 1):
            S = np.exp(gam[tt]) * S0
            for tau in range(1, tt + 1):
                c = axes[tau - 1]
                b = beta[0, tau - 1, h]
                col = np.exp(gam[tau]) * (1.0 - b) * S0[:, c] + b * v[0, tau - 1, h]
                S[:, c] = np.exp(gam[tt] - gam[tau]) * col
            assert _rel(out[0, tt - 1, h], S @ qh[0, tt - 1, 0]) < 1e-12
        assert _rel(st[0, h], S.T) < 1e-12


def pin_literal_matrices(run):
    """The definition evaluated with explicit d_k x d_k matrices (O(d^3) per token)."""
    q, k, v, g, beta, s0 = rand_case(5, n=2, t=16, h_qk=1, h_v=2, d_k=6, d_v=5)
    out, st = run(q, k, v, g, beta, s0, 1e-6)
    qh, kh = _unit(q, 1e-6), _unit(k, 1e-6)
    for b in range(2):
        for h in range(2):
            S = s0[b, h].T.copy()
            for tt in range(16):
                kk = kh[b, tt, 0][:, None]
                P = np.eye(6) - beta[b, tt, h] * (kk @ kk.T)
                S = np.exp(g[b, tt, h]) * (S @ P) + beta[b, tt, h] * (v[b, tt, h][:, None] @ kk.T)
                assert _rel(out[b, tt, h], S @ qh[b, tt, 0]) < 1e-12
            assert _rel(st[b, h], S.T) < 1e-12


def pin_chunked_equals_scan(run):
    """The re-blocked (UT/WY) evaluation equals the token scan, for chunk sizes that do
    and do not divide the length."""
    for t in (64, 37):
        q, k, v, g, beta, s0 = rand_case(6 + t, n=1, t=t, h_qk=1, h_v=2, d_k=16, d_v=16)
        out, st = run(q, k, v, g, beta, s0, 1e-6)
        for c in (1, 2, 4, 8, 16):
            o2, s2 = chunked(q, k, v, g, beta, s0, c, 1e-6)
            assert _rel(out, o2) < 1e-11, (t, c, _rel(out, o2))
            assert _rel(st, s2) < 1e-11, (t, c, _rel(st, s2))


def pin_segment_carry(run):
    """Processing a sequence in two calls with the state carried equals one call,
    bitwise (the recurrence is sequential; cutting it changes no operation)."""
    q, k, v, g, beta, s0 = rand_case(7, n=2, t=50, h_qk=2, h_v=4, d_k=8, d_v=8)
    out, st = run(q, k, v, g, beta, s0, 1e-6)
    cut = 19
    o1, s1 = run(q[:, :cut], k[:, :cut], v[:, :cut], g[:, :cut], beta[:, :cut], s0, 1e-6)
    o2, s2 = run(q[:, cut:], k[:, cut:], v[:, cut:], g[:, cut:], beta[:, cut:], s1, 1e-6)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), out)
    assert np.array_equal(s2, st)


def pin_linearity(run):
    """For fixed q, k, g, beta the map (S_0, V) -> (O, S_T) is linear."""
    q, k, v, g, beta, s0 = rand_case(8, t=20, d_k=8, d_v=8)
    _, _, v2, _, _, s02 = rand_case(9, t=20, d_k=8, d_v=8)
    o1, st1 = run(q, k, v, g, beta, s0, 1e-6)
    o2, st2 = run(q, k, v2, g, beta, s02, 1e-6)
    o3, st3 = run(q, k, 2.0 * v - 3.0 * v2, g, beta, 2.0 * s0 - 3.0 * s02, 1e-6)
    assert _rel(o3, 2.0 * o1 - 3.0 * o2) < 1e-12
    assert _rel(st3, 2.0 * st1 - 3.0 * st2) < 1e-12


def pin_column_independence(run):
    """A value channel j whose v and initial state column are zero stays exactly zero."""
    q, k, v, g, beta, s0 = rand_case(10, t=20, d_k=8, d_v=8)
    v[:, :, :, 3] = 0.0
    s0[:, :, :, 3] = 0.0
    out, st = run(q, k, v, g, beta, s0, 1e-6)
    assert np.all(out[:, :, :, 3] == 0.0) and np.all(st[:, :, :, 3] == 0.0)
    assert np.all(out[:, :, :, 2] != 0.0)


def pin_head_mapping(run):
    """V head h reads QK head h // (h_v / h_qk): each V head equals a one-head problem
    built from that QK head, bitwise."""
    q, k, v, g, beta, s0 = rand_case(11, n=1, t=12, h_qk=3, h_v=6, d_k=8, d_v=8)
    out, st = run(q, k, v, g, beta, s0, 1e-6)
    for h in range(6):
        m = h // 2
        o1, s1 = run(q[:, :, m:m + 1], k[:, :, m:m + 1], v[:, :, h:h + 1], g[:, :, h:h + 1],
                     beta[:, :, h:h + 1], s0[:, h:h + 1], 1e-6)
        assert np.array_equal(o1[:, :, 0], out[:, :, h])
        assert np.array_equal(s1[:, 0], st[:, h])


def pin_state_layout(run):
    """d_k != d_v, S_0 = 0, g = 0, beta = 1, k = 2 e_1 (so khat = e_1 exactly):
    S_1 = v e_1^T, stored transposed: state[1][j] = v_j and all else 0; with q = e_1 the
    output is v."""
    d_k, d_v = 3, 5
    q, k, v, g, beta, _ = rand_case(12, t=1, h_qk=1, h_v=1, d_k=d_k, d_v=d_v)
    k[:] = 0.0
    k[0, 0, 0, 1] = 2.0
    q[:] = 0.0
    q[0, 0, 0, 1] = 1.0
    g[:] = 0.0
    beta[:] = 1.0
    out, st = run(q, k, v, g, beta, None, 0.0)
    expect = np.zeros((d_k, d_v))
    expect[1] = v[0, 0, 0]
    assert np.array_equal(st[0, 0], expect)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0])


def pin_eps_placement(run):
    """l2_eps enters under the square root: k = e_1, eps = 3 gives khat = e_1 / 2."""
    q, k, v, g, beta, _ = rand_case(13, t=1, h_qk=1, h_v=1, d_k=4, d_v=4)
    k[:] = 0.0
    k[0, 0, 0, 0] = 1.0
    q[:] = 0.0
    q[0, 0, 0, 0] = 1.0
    g[:] = 0.0
    beta[:] = 1.0
    out, st = run(q, k, v, g, beta, None, 3.0)
    assert np.allclose(st[0, 0, 0], 0.5 * v[0, 0, 0], rtol=1e-15, atol=0)
    assert np.allclose(out[0, 0, 0], 0.25 * v[0, 0, 0], rtol=1e-15, atol=0)


def pin_scale_invariance(run):
    """With l2_eps = 0 only the directions of q and k matter."""
    q, k, v, g, beta, s0 = rand_case(14, t=20, d_k=8, d_v=8)
    o1, s1 = run(q, k, v, g, beta, s0, 0.0)
    o2, s2 = run(3.0 * q, 0.25 * k, v, g, beta, s0, 0.0)
    assert _rel(o2, o1) < 1e-13 and _rel(s2, s1) < 1e-13


PINS = [pin_identity, pin_decay_only, pin_retrieval, pin_orthonormal_keys,
        pin_literal_matrices, pin_chunked_equals_scan, pin_segment_carry, pin_linearity,
        pin_column_independence, pin_head_mapping, pin_state_layout, pin_eps_placement,
        pin_scale_invariance]
