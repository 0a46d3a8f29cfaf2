"""Pins of the oracle's prefix-cache snapshots (oracle.prefill_snapshots).

As for the speculative verify, identity conv taps (w[:, 0] = 1) give q, k, v
in closed form, so every snapshot can be checked against the closed-form
affine unroll of the delta rule at its position, its history against the
window entries, and chaining (a prefill started from a snapshot over the rest
of the request reproduces the whole request's final state and outputs) against
the oracle's own prefill.  Slot bookkeeping and errors are checked too.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from test_oracle_recurrence import affine_unroll
from test_oracle_spec import L2_EPS, NORM_EPS, closed_qkv


def case(seed, lens, interval, max_snaps, Hk=2, Hv=6, d=4):
    rng = np.random.default_rng(seed)
    nreq = len(lens)
    T = int(sum(lens))
    C = 2 * Hk * d + Hv * d
    num_slots = nreq * (max_snaps + 1) + 4
    perm = rng.permutation(num_slots)
    slot_ids = perm[:nreq]
    snaps = perm[nreq:nreq + nreq * max_snaps].reshape(nreq, max_snaps)
    w = np.zeros((C, 4))
    w[:, 0] = 1.0
    return dict(x=rng.standard_normal((T, C)), z=rng.standard_normal((T, Hv, d)),
                a=rng.standard_normal((T, Hv)), b=rng.standard_normal((T, Hv)), w=w,
                gamma=1.0 + 0.1 * rng.standard_normal(d),
                hist=rng.standard_normal((num_slots, C, 3)),
                state=rng.standard_normal((num_slots, Hv, d, d)) * 0.3,
                qsl=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64), slot_ids=slot_ids,
                snaps=snaps, hi=np.ones(nreq, np.uint8), Hk=Hk, Hv=Hv, d=d, interval=interval)


def run(c, snaps=None, interval=None, hi=None):
    return oracle.prefill_snapshots(
        c["x"], c["z"], c["a"], c["b"], c["w"], c["gamma"], c["hist"], c["state"], c["qsl"],
        c["slot_ids"], c["hi"] if hi is None else hi, c["snaps"] if snaps is None else snaps,
        c["interval"] if interval is None else interval, c["Hk"], c["Hv"], c["d"], c["d"],
        L2_EPS, NORM_EPS)


def test_snapshots_match_affine_unroll():
    c = case(21, [13, 4, 9, 0], interval=4, max_snaps=2)
    _, o, hist, state = run(c)
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
            np.testing.assert_allclose(state[c["slot_ids"][r], h], states[-1], rtol=0, atol=1e-12)
            for j in range(min((t1 - t0) // 4, 2)):   # request 0: positions 4, 8 (not 12)
                np.testing.assert_allclose(state[c["snaps"][r, j], h], states[4 * (j + 1) - 1],
                                           rtol=0, atol=1e-12)


def test_snapshot_history_and_untouched_slots():
    c = case(22, [11, 8, 3], interval=4, max_snaps=3)
    _, _, hist, state = run(c)
    written = set()
    for r, (t0, t1) in enumerate(zip(c["qsl"][:-1], c["qsl"][1:])):
        window = np.concatenate([c["hist"][c["slot_ids"][r]].T, c["x"][t0:t1]], axis=0)
        np.testing.assert_array_equal(hist[c["slot_ids"][r]], window[-3:].T)
        written.add(int(c["slot_ids"][r]))
        for j in range(min((t1 - t0) // 4, 3)):
            n = 4 * (j + 1)
            s = c["snaps"][r, j]
            written.add(int(s))
            np.testing.assert_array_equal(hist[s], window[n:n + 3].T)
    for s in range(c["state"].shape[0]):
        if s not in written:
            np.testing.assert_array_equal(state[s], c["state"][s])
            np.testing.assert_array_equal(hist[s], c["hist"][s])


def test_resuming_from_a_snapshot_reproduces_the_request():
    """Prefix caching: a later request that starts from snapshot j and runs the
    remaining tokens ends where the whole request ended, with the same outputs."""
    c = case(23, [20], interval=8, max_snaps=2)
    y, o, hist, state = run(c)
    for j in (0, 1):
        n = 8 * (j + 1)
        rest = slice(n, 20)
        s = c["snaps"][0, j]
        q2, k2, v2, h2 = oracle.conv1d_update(c["x"][rest], c["w"], hist, [0, 20 - n], [s], [1],
                                              c["Hk"], c["Hv"], c["d"], c["d"], L2_EPS)
        o2, st2 = oracle.gated_delta_rule(q2, k2, v2, c["a"][rest], c["b"][rest], state,
                                          [0, 20 - n], [s], [1])
        np.testing.assert_allclose(o2, o[rest], rtol=0, atol=1e-12)
        np.testing.assert_allclose(st2[s], state[c["slot_ids"][0]], rtol=0, atol=1e-12)
        np.testing.assert_array_equal(h2[s], hist[c["slot_ids"][0]])


def test_no_initial_state_and_exact_multiple():
    c = case(24, [8, 12], interval=4, max_snaps=3)
    hi = np.array([0, 1], np.uint8)
    _, _, hist, state = run(c, hi=hi)
    # request 0 starts from zero: its last snapshot (after 8 = all its tokens) is its final state
    np.testing.assert_array_equal(state[c["snaps"][0, 1]], state[c["slot_ids"][0]])
    np.testing.assert_array_equal(hist[c["snaps"][0, 1]], hist[c["slot_ids"][0]])
    c0 = dict(c)
    c0["state"] = c["state"].copy()
    c0["hist"] = c["hist"].copy()
    c0["state"][c["slot_ids"][0]] = 0.0
    c0["hist"][c["slot_ids"][0]] = 0.0
    _, _, hist0, state0 = run(c0)
    np.testing.assert_array_equal(state0[c["snaps"][0, 0]], state[c["snaps"][0, 0]])
    np.testing.assert_array_equal(hist0[c["snaps"][0, 0]], hist[c["snaps"][0, 0]])


def test_bad_snapshot_slots_raise():
    c = case(25, [9, 9], interval=4, max_snaps=2)
    bad = c["snaps"].copy()
    bad[1, 1] = bad[0, 0]
    with pytest.raises(ValueError):
        run(c, snaps=bad)
    bad = c["snaps"].copy()
    bad[0, 1] = c["slot_ids"][1]
    with pytest.raises(ValueError):
        run(c, snaps=bad)
    with pytest.raises(ValueError):
        run(c, interval=0)
