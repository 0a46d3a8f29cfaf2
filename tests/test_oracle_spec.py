"""Pins of the oracle's speculative multi-token verify (oracle.spec_verify).

With conv taps w[:, 0] = 1 and the other taps 0 the conv is the identity on the
current token, so q = normalize(SiLU(x_q)), k = normalize(SiLU(x_k)) and
v = SiLU(x_v) have closed forms; the checks below then hold position by
position without going through the oracle's own recurrence: the closed-form
affine unroll of the delta rule, the exact write S_j k_j = v_j at beta = 1, the
rank-1 write after decay, the identity at alpha = 1, beta = 0, and the history
as the last three entries of the window.  Slot bookkeeping (input slot kept,
unused slots untouched, aliasing position 0 onto the input slot, errors) is
checked on the same cases.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from test_oracle_recurrence import BIG, affine_unroll

L2_EPS = 1e-6
NORM_EPS = 1e-6


def silu(x):
    return x * expit(x)


def case(seed, lens, Hk=2, Hv=6, d=4, num_slots=None, a_val=None, b_val=None):
    rng = np.random.default_rng(seed)
    nreq = len(lens)
    T = int(sum(lens))
    C = 2 * Hk * d + Hv * d
    maxn = max(max(lens), 1)
    num_slots = num_slots or nreq * (maxn + 1) + 3
    perm = rng.permutation(num_slots)
    slot_ids = perm[:nreq]
    spec = perm[nreq:nreq + nreq * maxn].reshape(nreq, maxn)
    x = rng.standard_normal((T, C))
    z = rng.standard_normal((T, Hv, d))
    a = rng.standard_normal((T, Hv)) if a_val is None else np.full((T, Hv), a_val)
    b = rng.standard_normal((T, Hv)) if b_val is None else np.full((T, Hv), b_val)
    w = np.zeros((C, 4))
    w[:, 0] = 1.0  # identity conv: c_t = SiLU(x_t)
    gamma = 1.0 + 0.1 * rng.standard_normal(d)
    hist = rng.standard_normal((num_slots, C, 3))
    state = rng.standard_normal((num_slots, Hv, d, d)) * 0.3
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(x=x, z=z, a=a, b=b, w=w, gamma=gamma, hist=hist, state=state, qsl=qsl,
                slot_ids=slot_ids, spec=spec, hi=np.ones(nreq, np.uint8), Hk=Hk, Hv=Hv, d=d)


def run(c, spec=None, hi=None):
    return oracle.spec_verify(c["x"], c["z"], c["a"], c["b"], c["w"], c["gamma"], c["hist"],
                              c["state"], c["qsl"], c["slot_ids"],
                              c["spec"] if spec is None else spec,
                              c["hi"] if hi is None else hi, c["Hk"], c["Hv"], c["d"], c["d"],
                              L2_EPS, NORM_EPS)


def closed_qkv(c):
    """q, k, v of the identity conv, written out."""
    Hk, Hv, d = c["Hk"], c["Hv"], c["d"]
    s = silu(c["x"])
    T = s.shape[0]
    q = s[:, :Hk * d].reshape(T, Hk, d)
    k = s[:, Hk * d:2 * Hk * d].reshape(T, Hk, d)
    v = s[:, 2 * Hk * d:].reshape(T, Hv, d)
    q = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + L2_EPS)
    k = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + L2_EPS)
    return q, k, v


def test_every_position_matches_affine_unroll():
    c = case(11, [4, 1, 3, 0, 2])
    y, o, hist, state = run(c)
    q, k, v = closed_qkv(c)
    alpha = 1.0 / (1.0 + np.exp(c["a"]))
    beta = expit(c["b"])
    G = c["Hv"] // c["Hk"]
    for r, (t0, t1) in enumerate(zip(c["qsl"][:-1], c["qsl"][1:])):
        if t1 == t0:
            continue
        for h in range(c["Hv"]):
            o_ref, states = affine_unroll(c["state"][c["slot_ids"][r], h], q[t0:t1], k[t0:t1],
                                          v[t0:t1, h], alpha[t0:t1, h], beta[t0:t1, h], h // G)
            np.testing.assert_allclose(o[t0:t1, h], o_ref, rtol=0, atol=1e-12)
            for j in range(t1 - t0):
                np.testing.assert_allclose(state[c["spec"][r, j], h], states[j], rtol=0, atol=1e-12)


def test_beta1_writes_v_at_every_position():
    c = case(12, [5, 3], b_val=BIG)
    _, _, _, state = run(c)
    _, k, v = closed_qkv(c)
    alpha = 1.0 / (1.0 + np.exp(c["a"]))
    G = c["Hv"] // c["Hk"]
    for r, t0 in enumerate(c["qsl"][:-1]):
        prev = c["state"][c["slot_ids"][r]]
        for j in range(c["qsl"][r + 1] - t0):
            for h in range(c["Hv"]):
                S = state[c["spec"][r, j], h]
                kk = k[t0 + j, h // G]
                n2 = kk @ kk  # 1 up to the L2-norm epsilon
                # beta = 1: S k = |k|^2 v + (1 - |k|^2) alpha S_prev k, i.e. S k = v for |k| = 1
                ref = n2 * v[t0 + j, h] + (1.0 - n2) * alpha[t0 + j, h] * (prev[h] @ kk)
                np.testing.assert_allclose(S @ kk, ref, rtol=0, atol=1e-12)
                assert abs(1.0 - n2) < 1e-4
            prev = state[c["spec"][r, j]]


def test_rank1_write_after_decay_per_position():
    c = case(13, [4, 4])
    _, _, _, state = run(c)
    alpha = 1.0 / (1.0 + np.exp(c["a"]))
    for r, t0 in enumerate(c["qsl"][:-1]):
        prev = c["state"][c["slot_ids"][r]]
        for j in range(4):
            cur = state[c["spec"][r, j]]
            for h in range(c["Hv"]):
                dlt = cur[h] - alpha[t0 + j, h] * prev[h]
                sv = np.linalg.svd(dlt, compute_uv=False)
                assert sv[1] <= 1e-12 * max(sv[0], 1.0)
            prev = cur


def test_identity_gates_keep_the_input_state():
    c = case(14, [3, 2], a_val=-BIG, b_val=-BIG)
    _, o, _, state = run(c)
    q, _, _ = closed_qkv(c)
    G = c["Hv"] // c["Hk"]
    for r, t0 in enumerate(c["qsl"][:-1]):
        S0 = c["state"][c["slot_ids"][r]]
        for j in range(c["qsl"][r + 1] - t0):
            np.testing.assert_array_equal(state[c["spec"][r, j]], S0)
            for h in range(c["Hv"]):
                np.testing.assert_allclose(o[t0 + j, h], S0[h] @ q[t0 + j, h // G] / np.sqrt(c["d"]),
                                           atol=1e-14)


def test_history_per_position_and_untouched_slots():
    c = case(15, [4, 1, 0, 3])
    _, _, hist, state = run(c)
    written = set()
    for r, (t0, t1) in enumerate(zip(c["qsl"][:-1], c["qsl"][1:])):
        window = np.concatenate([c["hist"][c["slot_ids"][r]].T, c["x"][t0:t1]], axis=0)
        for j in range(t1 - t0):
            s = c["spec"][r, j]
            written.add(int(s))
            np.testing.assert_array_equal(hist[s], window[j + 1:j + 4].T)
    for s in range(c["state"].shape[0]):
        if s not in written:  # input slots included: read, never written
            np.testing.assert_array_equal(state[s], c["state"][s])
            np.testing.assert_array_equal(hist[s], c["hist"][s])


def test_no_initial_state_starts_from_zero():
    c = case(16, [3, 2])
    hi = np.array([0, 1], np.uint8)
    _, o, hist, state = run(c, hi=hi)
    c0 = dict(c)
    c0["state"] = c["state"].copy()
    c0["hist"] = c["hist"].copy()
    c0["state"][c["slot_ids"][0]] = 0.0
    c0["hist"][c["slot_ids"][0]] = 0.0
    _, o2, hist2, state2 = run(c0)
    np.testing.assert_array_equal(o, o2)
    for j in range(3):
        np.testing.assert_array_equal(state[c["spec"][0, j]], state2[c["spec"][0, j]])
        np.testing.assert_array_equal(hist[c["spec"][0, j]], hist2[c["spec"][0, j]])


def test_position0_may_alias_the_input_slot():
    c = case(17, [3, 2, 4])
    y, o, hist, state = run(c)
    spec = c["spec"].copy()
    spec[:, 0] = c["slot_ids"]
    y2, o2, hist2, state2 = run(c, spec=spec)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(y, y2)
    for r in range(3):
        for j in range(int(c["qsl"][r + 1] - c["qsl"][r])):
            np.testing.assert_array_equal(state2[spec[r, j]], state[c["spec"][r, j]])
            np.testing.assert_array_equal(hist2[spec[r, j]], hist[c["spec"][r, j]])


def test_single_token_equals_decode_step():
    c = case(18, [1, 1, 1])
    _, o, _, state = run(c)
    q, k, v = closed_qkv(c)
    o_d, pool_d = oracle.decode_step(q, k, v, c["a"], c["b"], c["state"], c["slot_ids"])
    np.testing.assert_allclose(o, o_d, rtol=0, atol=1e-14)
    for r in range(3):
        np.testing.assert_allclose(state[c["spec"][r, 0]], pool_d[c["slot_ids"][r]], atol=1e-15)


def test_bad_metadata_raises():
    c = case(19, [3, 2])
    spec = c["spec"].copy()
    spec[1, 0] = spec[0, 1]
    with pytest.raises(ValueError):
        run(c, spec=spec)
    spec = c["spec"].copy()
    spec[1, 1] = c["slot_ids"][0]  # another request's input slot
    with pytest.raises(ValueError):
        run(c, spec=spec)
    with pytest.raises(ValueError):
        run(c, spec=c["spec"][:, :2])  # fewer positions than tokens
