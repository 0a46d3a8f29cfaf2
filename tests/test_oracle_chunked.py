"""The chunkwise form of the gated delta rule (the algebra the GPU prefill runs)
against the oracle's sequential recurrence, on the CPU in fp64.

For a chunk of C tokens with state S0 (dv x dk), cumulative log-decay
G_t = sum_{s<=t} log alpha_s and the chunk's q, k, v, beta:
  (I + A) Delta = diag(beta) (V - diag(e^G) K S0^T),  A_ts = beta_t e^{G_t-G_s} k_t.k_s (s < t)
  O = diag(e^G) Q S0^T + P Delta,                      P_ts = e^{G_t-G_s} q_t.k_s (s <= t)
  S_C = e^{G_C} S0 + (diag(e^{G_C-G}) Delta)^T K
with o scaled by 1/sqrt(dk).  Written here from the recurrence (tutorial page,
section 01, per-layer operator table) by unrolling it over a chunk; it must
reach the sequential result up to rounding for any chunk length, including
lengths that do not divide T; an off-by-one in the triangular masks or the
chunk's decay applied in the wrong place fails it.
"""
import numpy as np
import pytest

from test_oracle_recurrence import rand_case, run1


def chunked_delta_rule(q, k, v, a, b, S0, C):
    """One request, every value head, chunk length C; returns o [T,Hv,dv] and
    the final state [Hv,dv,dk]."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1:]
    group = Hv // Hk
    logalpha = -np.logaddexp(0.0, a)        # log exp(-softplus(a))
    beta = 1.0 / (1.0 + np.exp(-b))
    o = np.zeros((T, Hv, dv))
    S = S0.copy()
    for h in range(Hv):
        kh = h // group
        Sh = S[h]
        for c0 in range(0, T, C):
            c1 = min(T, c0 + C)
            Q, K, V = q[c0:c1, kh], k[c0:c1, kh], v[c0:c1, h]
            bt = beta[c0:c1, h]
            G = np.cumsum(logalpha[c0:c1, h])
            D = np.exp(G[:, None] - G[None, :])          # e^{G_t - G_s}
            n = c1 - c0
            strict = np.tril(np.ones((n, n)), -1)
            A = strict * bt[:, None] * D * (K @ K.T)
            rhs = bt[:, None] * (V - np.exp(G)[:, None] * (K @ Sh.T))
            Delta = np.linalg.solve(np.eye(n) + A, rhs)
            P = np.tril(np.ones((n, n))) * D * (Q @ K.T)
            o[c0:c1, h] = (np.exp(G)[:, None] * (Q @ Sh.T) + P @ Delta) / np.sqrt(dk)
            Sh = np.exp(G[-1]) * Sh + (np.exp(G[-1] - G)[:, None] * Delta).T @ K
        S[h] = Sh
    return o, S


@pytest.mark.parametrize("C", [1, 3, 8, 32, 64])
def test_chunked_form_equals_sequential(C):
    rng = np.random.default_rng(100 + C)
    T, Hk, Hv, dk, dv = 77, 2, 6, 16, 12      # C does not divide T (except C = 1)
    q, k, v, a, b = rand_case(rng, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((Hv, dv, dk)) * 0.3
    o_ref, st_ref = run1(q, k, v, a, b, S0)
    o, S = chunked_delta_rule(q, k, v, a, b, S0, C)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, st_ref[0], rtol=0, atol=1e-12)


def test_chunked_form_strong_decay_and_write():
    """Gates near saturation (alpha -> 0 or 1, beta -> 0 or 1) over a chunk of 32."""
    rng = np.random.default_rng(7)
    T, Hk, Hv, dk, dv = 40, 1, 3, 8, 8
    q, k, v, a, b = rand_case(rng, T, Hk, Hv, dk, dv)
    a = a * 6.0
    b = b * 6.0
    S0 = rng.standard_normal((Hv, dv, dk))
    o_ref, st_ref = run1(q, k, v, a, b, S0)
    o, S = chunked_delta_rule(q, k, v, a, b, S0, 32)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(S, st_ref[0], rtol=0, atol=1e-10)


def test_chunked_form_catches_planted_mistakes():
    """The comparison is sharp: an inclusive diagonal in A (a token's own write
    counted twice) or the decay of a whole chunk applied to the initial state's
    outputs at the chunk end instead of per token breaks the agreement."""
    rng = np.random.default_rng(8)
    T, Hk, Hv, dk, dv = 20, 1, 2, 8, 8
    q, k, v, a, b = rand_case(rng, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((Hv, dv, dk))
    o_ref, _ = run1(q, k, v, a, b, S0)
    good = chunked_variant(q, k, v, a, b, S0, 8)
    assert np.max(np.abs(good - o_ref)) < 1e-12
    assert np.max(np.abs(chunked_variant(q, k, v, a, b, S0, 8, a_diag=0) - o_ref)) > 1e-3
    assert np.max(np.abs(chunked_variant(q, k, v, a, b, S0, 8, chunk_end_decay=True) - o_ref)) > 1e-3


def chunked_variant(q, k, v, a, b, S0, C, a_diag=-1, chunk_end_decay=False):
    """chunked_delta_rule's outputs with one step optionally altered."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1:]
    logalpha = -np.logaddexp(0.0, a)
    beta = 1.0 / (1.0 + np.exp(-b))
    o = np.zeros((T, Hv, dv))
    for h in range(Hv):
        kh = h // (Hv // Hk)
        Sh = S0[h].copy()
        for c0 in range(0, T, C):
            c1 = min(T, c0 + C)
            Q, K, V = q[c0:c1, kh], k[c0:c1, kh], v[c0:c1, h]
            bt = beta[c0:c1, h]
            G = np.cumsum(logalpha[c0:c1, h])
            D = np.exp(G[:, None] - G[None, :])
            n = c1 - c0
            A = np.tril(np.ones((n, n)), a_diag) * bt[:, None] * D * (K @ K.T)
            rhs = bt[:, None] * (V - np.exp(G)[:, None] * (K @ Sh.T))
            Delta = np.linalg.solve(np.eye(n) + A, rhs)
            P = np.tril(np.ones((n, n))) * D * (Q @ K.T)
            gq = np.full(n, np.exp(G[-1])) if chunk_end_decay else np.exp(G)
            o[c0:c1, h] = (gq[:, None] * (Q @ Sh.T) + P @ Delta) / np.sqrt(dk)
            Sh = np.exp(G[-1]) * Sh + (np.exp(G[-1] - G)[:, None] * Delta).T @ K
    return o
