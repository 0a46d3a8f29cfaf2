"""Pins of the oracle's conv1d, SiLU, L2 norm, RMSNorm, gated norm, residual and
layer composition against library routines, closed forms and the worked
examples printed on the tutorial page (section 01 LAYER-BY-LAYER)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle


def packed(rng, lens, C, taps=4, nslots=None):
    T = sum(lens)
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, taps))
    nslots = nslots or len(lens)
    hist = rng.standard_normal((nslots, C, taps - 1))
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return x, w, hist, qsl


def test_conv_matches_numpy_convolve():
    rng = np.random.default_rng(0)
    lens = [7, 1, 2, 5]
    C = 6
    x, w, hist, qsl = packed(rng, lens, C)
    slots = [2, 0, 3, 1]
    c, _ = oracle.conv1d_silu(x, w, hist, qsl, slots)
    for r, s in enumerate(slots):
        for ch in range(C):
            window = np.concatenate([hist[s, ch], x[qsl[r]:qsl[r + 1], ch]])
            y = np.convolve(window, w[ch], mode="valid")  # sum_i w_i x_{t-i}
            ref = torch.nn.functional.silu(torch.from_numpy(y)).numpy()
            np.testing.assert_allclose(c[qsl[r]:qsl[r + 1], ch], ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("lag", [0, 1, 2, 3])
def test_conv_one_hot_tap_is_a_shift(lag):
    rng = np.random.default_rng(1)
    lens = [6]
    C = 3
    x, _, hist, qsl = packed(rng, lens, C)
    w = np.zeros((C, 4))
    w[:, lag] = 1.0
    c, _ = oracle.conv1d_silu(x, w, hist, qsl, [0])
    window = np.concatenate([hist[0].T, x])  # [3 + T, C]
    shifted = window[3 - lag: 3 - lag + 6]
    np.testing.assert_allclose(c, shifted / (1 + np.exp(-shifted)), rtol=1e-15)


def test_conv_history_writeback_and_zero_start():
    rng = np.random.default_rng(2)
    lens = [1, 2, 5, 0]
    C = 4
    x, w, hist, qsl = packed(rng, lens, C, nslots=5)
    slots = [4, 1, 0, 2]
    has_init = [1, 1, 0, 1]
    c, new = oracle.conv1d_silu(x, w, hist, qsl, slots, has_init)
    # L = 1: [h-2, h-1, x0]
    np.testing.assert_array_equal(new[4], np.stack([hist[4, :, 1], hist[4, :, 2], x[0]], 1))
    # L = 2: [h-1, x0, x1]
    np.testing.assert_array_equal(new[1], np.stack([hist[1, :, 2], x[1], x[2]], 1))
    # L = 5: last three rows
    np.testing.assert_array_equal(new[0], x[5:8].T)
    # empty request and unused slot untouched
    np.testing.assert_array_equal(new[2], hist[2])
    np.testing.assert_array_equal(new[3], hist[3])
    # has_initial = 0 reads zeros, not the slot
    c0, _ = oracle.conv1d_silu(x[3:8], w, np.zeros((1, C, 3)), [0, 5], [0])
    np.testing.assert_allclose(c[3:8], c0, rtol=0, atol=0)


def test_conv_no_cross_request_mixing():
    rng = np.random.default_rng(3)
    lens = [3, 4]
    C = 5
    x, w, hist, qsl = packed(rng, lens, C)
    c, _ = oracle.conv1d_silu(x, w, hist, qsl, [0, 1])
    c1, _ = oracle.conv1d_silu(x[3:], w, hist[1:2], [0, 4], [0])
    np.testing.assert_array_equal(c[3:], c1)


def test_silu_and_l2norm_textbook():
    y = np.linspace(-30, 30, 101)
    np.testing.assert_allclose(oracle.silu(y), torch.nn.functional.silu(torch.from_numpy(y)).numpy(),
                               rtol=1e-14, atol=1e-300)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 3, 16))
    n = oracle.l2norm(x, 0.0)
    np.testing.assert_allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(n, torch.nn.functional.normalize(torch.from_numpy(x), dim=-1).numpy(),
                               rtol=1e-14)
    assert np.all(oracle.l2norm(np.zeros((2, 8)), 1e-6) == 0)


def test_conv1d_update_split_order():
    """q | k | v split in the in-projection's Q0, K0, V0 order, q and k normalised per head."""
    rng = np.random.default_rng(5)
    Hk, Hv, dk, dv = 2, 4, 3, 5
    C = 2 * Hk * dk + Hv * dv
    x, w, hist, qsl = packed(rng, [6], C)
    q, k, v, _ = oracle.conv1d_update(x, w, hist, qsl, [0], [1], Hk, Hv, dk, dv, 0.0)
    c, _ = oracle.conv1d_silu(x, w, hist, qsl, [0])
    np.testing.assert_allclose(q * np.linalg.norm(c[:, :6].reshape(6, 2, 3), axis=-1, keepdims=True),
                               c[:, :6].reshape(6, 2, 3), rtol=1e-14)
    np.testing.assert_allclose(k[:, 1] / np.linalg.norm(k[:, 1], axis=-1, keepdims=True),
                               c[:, 9:12] / np.linalg.norm(c[:, 9:12], axis=-1, keepdims=True), rtol=1e-14)
    np.testing.assert_array_equal(v, c[:, 12:].reshape(6, Hv, dv))


def test_rmsnorm_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "rmsnorm_worked_example.json")) as f:
        g = json.load(f)
    x = np.array(g["input"])
    y = oracle.rmsnorm(x, np.ones(4), 1e-6)
    np.testing.assert_allclose(y, g["output"], atol=g["print_precision"])
    # a mean-subtracted LayerNorm does not reproduce the printed row
    ln = (x - x.mean()) / np.sqrt(x.var() + 1e-6)
    assert np.abs(ln - np.array(g["output"])).max() > 1e-2


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((7, 33))
    g = rng.standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 1e-6), ref.numpy(), rtol=1e-13)


def test_gated_norm_per_value_head():
    rng = np.random.default_rng(7)
    T, Hv, dv = 5, 3, 8
    o = rng.standard_normal((T, Hv, dv)) * rng.uniform(0.1, 10, (T, Hv, 1))
    z = rng.standard_normal((T, Hv, dv))
    g = rng.uniform(0.5, 1.5, dv)
    y = oracle.gated_norm(o, z, g, 1e-6).reshape(T, Hv, dv)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (dv,), torch.from_numpy(g), eps=1e-6) \
        * torch.nn.functional.silu(torch.from_numpy(z))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13)
    # each head is normalised on its own: a whole-row norm would differ
    row = oracle.rmsnorm(o.reshape(T, -1), np.tile(g, Hv), 1e-6).reshape(T, Hv, dv) * oracle.silu(z)
    assert np.abs(row - y).max() > 1e-2


def test_residual_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "residual_worked_example.json")) as f:
        g = json.load(f)
    y = oracle.residual_add(oracle.residual_add(g["x_in"], g["delta_mix"]), g["delta_ffn"])
    tol = g["print_precision"]
    np.testing.assert_allclose(y, g["x_out"], atol=tol)
    assert abs(np.linalg.norm(g["x_in"]) - g["norm_in"]) < tol
    assert abs(np.linalg.norm(y) - g["norm_out"]) < tol
    d = np.add(g["delta_mix"], g["delta_ffn"])
    assert abs(np.linalg.norm(d) - g["norm_delta"]) < tol


def test_layer_composition_and_residual_identity():
    rng = np.random.default_rng(8)
    Hk, Hv, dk, dv, hidden = 1, 2, 4, 3, 10
    C = 2 * Hk * dk + Hv * dv
    lens = [4, 1]
    T = 5
    X = rng.standard_normal((T, hidden))
    gi = rng.uniform(0.5, 1.5, hidden)
    Wqkvz = rng.standard_normal((hidden, C + Hv * dv)) * 0.3
    Wba = rng.standard_normal((hidden, 2 * Hv)) * 0.3
    cw = rng.standard_normal((C, 4))
    go = rng.uniform(0.5, 1.5, dv)
    Wo = rng.standard_normal((Hv * dv, hidden)) * 0.3
    hist = rng.standard_normal((2, C, 3))
    st = rng.standard_normal((2, Hv, dv, dk))
    qsl = [0, 4, 5]
    Y, nh, ns, it = oracle.gdn_layer(X, gi, Wqkvz, Wba, cw, go, Wo, hist, st, qsl, [1, 0], [0, 1],
                                     Hk, Hv, dk, dv, 1e-6, 1e-6)
    U = oracle.rmsnorm(X, gi, 1e-6)
    P = U @ Wqkvz
    q, k, v, nh2 = oracle.conv1d_update(P[:, :C], cw, hist, qsl, [1, 0], [0, 1], Hk, Hv, dk, dv, 1e-6)
    ba = U @ Wba
    o, ns2 = oracle.gated_delta_rule(q, k, v, ba[:, Hv:], ba[:, :Hv], st, qsl, [1, 0], [0, 1])
    y = oracle.gated_norm(o, P[:, C:].reshape(T, Hv, dv), go, 1e-6)
    np.testing.assert_allclose(Y, X + y @ Wo, rtol=1e-13)
    np.testing.assert_array_equal(nh, nh2)
    np.testing.assert_array_equal(ns, ns2)
    Y0, *_ = oracle.gdn_layer(X, gi, Wqkvz, Wba, cw, go, np.zeros_like(Wo), hist, st, qsl, [1, 0],
                              [0, 1], Hk, Hv, dk, dv, 1e-6, 1e-6)
    np.testing.assert_array_equal(Y0, X)


def test_round_bf16_matches_library_rounding():
    """The bf16 state rounding: round to nearest, ties to even, checked against
    torch's float32 -> bfloat16 conversion (a library rounding routine) on random
    values, values exactly halfway between two bf16 numbers, and specials."""
    import torch
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        [0.0, -0.0, np.inf, -np.inf, 1e-40, -3.4e38]])
    # halfway cases: a bf16 value plus half of its ulp (ties go to the even neighbour)
    base = rng.standard_normal(2000).astype(np.float32)
    bits = base.view(np.uint32) & np.uint32(0xFFFF0000)
    halfway = (bits | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    for v in (x, halfway):
        v32 = v.astype(np.float32)  # float32 inputs: one rounding on both sides
        ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(oracle.round_bf16(v32.astype(np.float64)), ref)
    assert np.isnan(oracle.round_bf16(np.array([np.nan]))[0])
    # round-tripping a bf16 value is the identity
    y = oracle.round_bf16(x[:1000])
    np.testing.assert_array_equal(oracle.round_bf16(y), y)
