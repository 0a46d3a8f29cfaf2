"""Pins of the oracle's gated delta rule against facts that do not come from the
oracle itself: a closed-form unroll, special cases with known answers, structural
invariants stated on the pages, and the GDN state-lab trace the tutorial page
prints (section 03 MEMORY LABS)."""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle

BIG = 1000.0  # |raw gate| that saturates exp/sigmoid exactly in fp64


def rand_case(rng, T, Hk, Hv, dk, dv, unit_k=True):
    q = rng.standard_normal((T, Hk, dk))
    k = rng.standard_normal((T, Hk, dk))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, dv))
    a = rng.standard_normal((T, Hv))
    b = rng.standard_normal((T, Hv))
    return q, k, v, a, b


def run1(q, k, v, a, b, S0=None, has_init=1):
    """One request in slot 0."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1:]
    pool = np.zeros((1, Hv, dv, dk)) if S0 is None else S0[None].copy()
    return oracle.gated_delta_rule(q, k, v, a, b, pool, [0, T], [0], [has_init])


def affine_unroll(S0, q, k, v, alpha, beta, kh):
    """Closed form of the recurrence for one value head: with
    M_t = alpha_t (I - beta_t k_t k_t^T) and N_t = beta_t v_t k_t^T,
    S_t = S0 M_1...M_t + sum_s N_s M_{s+1}...M_t, and o_t = S_t q_t / sqrt(dk)."""
    T = q.shape[0]
    dk = q.shape[-1]
    M = [alpha[t] * (np.eye(dk) - beta[t] * np.outer(k[t, kh], k[t, kh])) for t in range(T)]
    N = [beta[t] * np.outer(v[t], k[t, kh]) for t in range(T)]
    outs, states = [], []
    for t in range(T):
        prod = np.eye(dk)
        for m in M[: t + 1]:
            prod = prod @ m
        S = S0 @ prod
        for s in range(t + 1):
            tail = np.eye(dk)
            for m in M[s + 1: t + 1]:
                tail = tail @ m
            S = S + N[s] @ tail
        states.append(S)
        outs.append(S @ q[t, kh] / np.sqrt(dk))
    return np.array(outs), states


@pytest.mark.parametrize("dk,dv", [(3, 5), (4, 4), (6, 2)])
def test_brute_force_affine_unroll(dk, dv):
    rng = np.random.default_rng(7)
    T, Hk, Hv = 6, 2, 6
    q, k, v, a, b = rand_case(rng, T, Hk, Hv, dk, dv, unit_k=False)
    S0 = rng.standard_normal((Hv, dv, dk))
    o, pool = run1(q, k, v, a, b, S0)
    alpha = np.exp(-np.log1p(np.exp(a)))
    beta = expit(b)
    for h in range(Hv):
        o_ref, states = affine_unroll(S0[h], q, k, v[:, h], alpha[:, h], beta[:, h], h // 3)
        np.testing.assert_allclose(o[:, h], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(pool[0, h], states[-1], rtol=0, atol=1e-12)


def test_identity_when_alpha1_beta0():
    rng = np.random.default_rng(1)
    T, dk, dv = 9, 5, 7
    q, k, v, _, _ = rand_case(rng, T, 1, 3, dk, dv)
    S0 = rng.standard_normal((3, dv, dk))
    a = np.full((T, 3), -BIG)  # softplus -> 0, alpha = 1
    b = np.full((T, 3), -BIG)  # beta = 0
    o, pool = run1(q, k, v, a, b, S0)
    np.testing.assert_array_equal(pool[0], S0)
    for h in range(3):
        np.testing.assert_allclose(o[:, h], q[:, 0] @ S0[h].T / np.sqrt(dk), atol=1e-14)


def test_beta1_unit_k_stores_v_exactly():
    """With beta = 1 and |k| = 1 the delta write makes S_t k_t = v_t."""
    rng = np.random.default_rng(2)
    T, dk, dv = 12, 8, 5
    q, k, v, a, _ = rand_case(rng, T, 1, 1, dk, dv)
    b = np.full((T, 1), BIG)
    S = rng.standard_normal((dv, dk))
    for t in range(T):
        _, pool = run1(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], S[None])
        S = pool[0, 0]
        np.testing.assert_allclose(S @ k[t, 0], v[t, 0], atol=1e-13)


def test_alpha0_forgets_everything():
    rng = np.random.default_rng(3)
    T, dk, dv = 4, 6, 3
    q, k, v, _, b = rand_case(rng, T, 1, 2, dk, dv)
    a = np.full((T, 2), BIG)  # alpha = exp(-1000) = 0
    S0 = rng.standard_normal((2, dv, dk))
    _, pool = run1(q, k, v, a, b, S0)
    beta = expit(b[-1])
    for h in range(2):
        np.testing.assert_allclose(pool[0, h], beta[h] * np.outer(v[-1, h], k[-1, 0]), atol=1e-14)


def test_beta0_pure_decay_and_zero_qk():
    rng = np.random.default_rng(4)
    T, dk, dv = 10, 4, 4
    q, k, v, a, _ = rand_case(rng, T, 1, 3, dk, dv)
    S0 = rng.standard_normal((3, dv, dk))
    alpha = np.exp(-np.logaddexp(0, a))
    b = np.full((T, 3), -BIG)
    _, pool = run1(q, k, v, a, b, S0)
    for h in range(3):
        np.testing.assert_allclose(pool[0, h], np.prod(alpha[:, h]) * S0[h], rtol=1e-13)
    # q = k = 0: the write vanishes whatever beta is, and the read is zero
    z = np.zeros_like(q)
    o, pool = run1(z, z, v, a, rng.standard_normal((T, 3)), S0)
    assert np.all(o == 0)
    for h in range(3):
        np.testing.assert_allclose(pool[0, h], np.prod(alpha[:, h]) * S0[h], rtol=1e-13)


def test_write_after_decay_is_rank_one():
    """S_t - alpha_t S_{t-1} = beta_t e_t k_t^T has rank <= 1."""
    rng = np.random.default_rng(5)
    T, dk, dv = 8, 6, 5
    q, k, v, a, b = rand_case(rng, T, 1, 1, dk, dv)
    alpha = np.exp(-np.logaddexp(0, a))
    S = rng.standard_normal((1, 1, dv, dk))
    for t in range(T):
        prev = S[0, 0].copy()
        _, S = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], S, [0])
        sv = np.linalg.svd(S[0, 0] - alpha[t, 0] * prev, compute_uv=False)
        assert sv[1] < 1e-12 * max(1.0, sv[0])


def test_split_equals_whole_and_decode_equals_prefill():
    rng = np.random.default_rng(6)
    T, dk, dv = 13, 4, 6
    q, k, v, a, b = rand_case(rng, T, 2, 4, dk, dv)
    S0 = rng.standard_normal((4, dv, dk))
    o_all, p_all = run1(q, k, v, a, b, S0)
    o1, p1 = run1(q[:5], k[:5], v[:5], a[:5], b[:5], S0)
    o2, p2 = run1(q[5:], k[5:], v[5:], a[5:], b[5:], p1[0])
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(p2, p_all, rtol=0, atol=1e-13)
    pool = S0[None].copy()
    outs = []
    for t in range(T):
        o, pool = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], pool, [0])
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs), o_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(pool, p_all, rtol=0, atol=1e-13)


def test_state_shape_independent_of_length():
    """The state-shape calculator has no sequence-length input (dispatch page, step 5)."""
    rng = np.random.default_rng(8)
    shapes = set()
    for T in (1, 7, 40):
        q, k, v, a, b = rand_case(rng, T, 2, 6, 4, 3)
        _, pool = run1(q, k, v, a, b)
        shapes.add(pool.shape)
    assert shapes == {(1, 6, 3, 4)}


def test_contiguous_key_head_groups():
    """Value head h reads key head h // (Hv/Hk): the 4-way tensor-parallel table
    keeps key heads 0-3 with value heads 0-11 on one rank.  Replicating each key
    head explicitly for its value heads must give the same result."""
    rng = np.random.default_rng(9)
    T, Hk, Hv, dk, dv = 7, 2, 6, 4, 4
    q, k, v, a, b = rand_case(rng, T, Hk, Hv, dk, dv)
    o, pool = run1(q, k, v, a, b)
    qx = np.repeat(q, Hv // Hk, axis=1)
    kx = np.repeat(k, Hv // Hk, axis=1)
    o2, pool2 = run1(qx, kx, v, a, b)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(pool, pool2)
    # an interleaved map would differ
    qi = np.tile(q, (1, Hv // Hk, 1))
    ki = np.tile(k, (1, Hv // Hk, 1))
    o3, _ = run1(qi, ki, v, a, b)
    assert np.abs(o3 - o).max() > 1e-3


def test_varlen_slots_no_mixing():
    rng = np.random.default_rng(10)
    Hk, Hv, dk, dv = 1, 3, 4, 5
    lens = [5, 0, 1, 9]
    T = sum(lens)
    q, k, v, a, b = rand_case(rng, T, Hk, Hv, dk, dv)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = [3, 0, 5, 1]
    has_init = [1, 1, 0, 1]
    pool0 = rng.standard_normal((6, Hv, dv, dk))
    o, pool = oracle.gated_delta_rule(q, k, v, a, b, pool0, qsl, slots, has_init)
    # untouched slots: 2, 4 (unused) and 0 (empty request)
    for s in (0, 2, 4):
        np.testing.assert_array_equal(pool[s], pool0[s])
    for r, (L, s, hi) in enumerate(zip(lens, slots, has_init)):
        if L == 0:
            continue
        sl = slice(qsl[r], qsl[r + 1])
        o_r, p_r = run1(q[sl], k[sl], v[sl], a[sl], b[sl], pool0[s], has_init=hi)
        np.testing.assert_array_equal(o[sl], o_r)
        np.testing.assert_array_equal(pool[s], p_r[0])
    # has_initial = 0 ignores whatever the slot held
    sl = slice(qsl[2], qsl[3])
    o_z, _ = run1(q[sl], k[sl], v[sl], a[sl], b[sl], None)
    np.testing.assert_array_equal(o[sl], o_z)


def test_metadata_errors():
    rng = np.random.default_rng(11)
    q, k, v, a, b = rand_case(rng, 4, 1, 1, 2, 2)
    pool = np.zeros((2, 1, 2, 2))
    with pytest.raises(ValueError):
        oracle.gated_delta_rule(q, k, v, a, b, pool, [0, 2, 4], [1, 1])
    with pytest.raises(ValueError):
        oracle.gated_delta_rule(q, k, v, a, b, pool, [0, 3, 2], [0, 1])
    with pytest.raises(ValueError):
        oracle.gated_delta_rule(q, k, v, a, b, pool, [0, 4], [2])
    with pytest.raises(ValueError):
        oracle.gated_delta_rule(q, k, v, a, b, pool, [0, 3], [0])


def test_gates_closed_forms():
    a = np.array([-50.0, -3.0, 0.0, 0.7, 3.0, 40.0])
    alpha, beta = oracle.gates(a, a)
    # exp(-log(1 + e^a)) = 1 / (1 + e^a) = sigmoid(-a)
    np.testing.assert_allclose(alpha, expit(-a), rtol=1e-14)
    np.testing.assert_allclose(beta, expit(a), rtol=1e-14)
    assert alpha[2] == 0.5 and beta[2] == 0.5
    al, be = oracle.gates(np.array([BIG, -BIG]), np.array([BIG, -BIG]))
    assert list(al) == [0.0, 1.0] and list(be) == [1.0, 0.0]


def test_gdn_lab_trace(golden_dir):
    """Reproduce the GDN state lab's printed 2x2 trace (alpha = 0.78).  The page
    prints no k, v, beta; each step's rank-1 write D_t = S_t - 0.78 S_{t-1} is
    read off the printed states (its best rank-1 part sigma u w^T), and the step
    is fed k_t = w, beta_t = 1, v_t = sigma u + 0.78 S_{t-1} k_t, i.e. the value
    whose error against the DECAYED state is sigma u.  The oracle must then land
    on the printed states to print precision (plus carried rounding)."""
    with open(os.path.join(golden_dir, "gdn_lab_trace.json")) as f:
        g = json.load(f)
    alpha = g["alpha"]
    printed = np.array(g["states"]).reshape(-1, 2, 2)
    a_raw = np.log(1.0 / alpha - 1.0)  # exp(-softplus(a)) = 1/(1+e^a) = alpha
    S = np.zeros((1, 1, 2, 2))
    prev_printed = np.zeros((2, 2))
    for t in range(printed.shape[0]):
        D = printed[t] - alpha * prev_printed
        U, sv, Vt = np.linalg.svd(D)
        kt = Vt[0]
        vt = sv[0] * U[:, 0] + alpha * S[0, 0] @ kt
        o, S = oracle.decode_step(np.zeros((1, 1, 2)), kt.reshape(1, 1, 2), vt.reshape(1, 1, 2),
                                  np.array([[a_raw]]), np.array([[BIG]]), S, [0])
        assert np.abs(S[0, 0] - printed[t]).max() < 0.02
        prev_printed = printed[t]
    # the undecayed-read variant (e = v - S_{t-1} k) misses the printed trace
    S_bad = np.zeros((2, 2))
    prev_printed = np.zeros((2, 2))
    worst = 0.0
    for t in range(printed.shape[0]):
        D = printed[t] - alpha * prev_printed
        U, sv, Vt = np.linalg.svd(D)
        kt = Vt[0]
        vt = sv[0] * U[:, 0] + alpha * S_bad @ kt
        S_bad = alpha * S_bad + np.outer(vt - S_bad @ kt, kt)
        worst = max(worst, np.abs(S_bad - printed[t]).max())
        prev_printed = printed[t]
    assert worst > 0.05
