"""Pins of the GQA decode oracle (oracle.rope_partial, oracle.gqa_decode_paged).

The rotation is checked against complex multiplication by e^{i angle} (a
different formulation), against its group and relative-position properties,
and on unit vectors whose image is known (pair 0 turns by the position in
radians).  The attention is checked against a dense computation written
independently (contiguous keys gathered by hand, scipy's softmax), against
closed forms (one position gives v; equal keys give the mean of the values;
a zero gate halves the output), against invariance under a relocation of the
physical pages, and against the head sharing the pages print (query head 7
reads key/value head 1).
"""
import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from oracle.gqa import _check_paged

RD = 64
THETA = 10000.0


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 256))
    pos = np.array([0, 1, 7, 4095, 131071])
    got = oracle.rope_partial(x, pos, RD, THETA)
    zc = (x[:, :, :32] + 1j * x[:, :, 32:64]) * np.exp(
        1j * pos[:, None, None] * THETA ** (-np.arange(0, RD, 2) / RD)[None, None, :])
    # angles reach 1.3e5 rad, where one fp64 ulp of the angle is 1.5e-11
    np.testing.assert_allclose(got[:, :, :32], zc.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(got[:, :, 32:64], zc.imag, rtol=0, atol=1e-9)
    np.testing.assert_array_equal(got[:, :, 64:], x[:, :, 64:])   # partial: 192 dims untouched
    np.testing.assert_array_equal(got[0], x[0])                   # position 0: identity


def test_rope_unit_vectors_and_frequencies():
    e0 = np.zeros((1, 1, 256))
    e0[0, 0, 0] = 1.0
    for p in (1, 3, 1000):
        r = oracle.rope_partial(e0, [p], RD, THETA)[0, 0]
        assert abs(r[0] - np.cos(p)) < 1e-15 and abs(r[32] - np.sin(p)) < 1e-15   # frequency 1
        assert np.count_nonzero(r) == 2
    e31 = np.zeros((1, 1, 256))
    e31[0, 0, 63] = 1.0                       # second member of the slowest pair
    r = oracle.rope_partial(e31, [1000], RD, THETA)[0, 0]
    ang = 1000 * THETA ** (-62 / 64)
    assert abs(r[63] - np.cos(ang)) < 1e-15 and abs(r[31] + np.sin(ang)) < 1e-15


def test_rope_group_and_relative_properties():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 256))
    k = rng.standard_normal((1, 2, 256))
    a = oracle.rope_partial(oracle.rope_partial(q, [17], RD, THETA), [25], RD, THETA)
    np.testing.assert_allclose(a, oracle.rope_partial(q, [42], RD, THETA), rtol=0, atol=1e-12)
    d1 = np.sum(oracle.rope_partial(q, [100], RD, THETA) * oracle.rope_partial(k, [60], RD, THETA))
    d2 = np.sum(oracle.rope_partial(q, [540], RD, THETA) * oracle.rope_partial(k, [500], RD, THETA))
    assert abs(d1 - d2) < 1e-10
    np.testing.assert_allclose(np.linalg.norm(oracle.rope_partial(q, [77], RD, THETA), axis=-1),
                               np.linalg.norm(q, axis=-1), rtol=1e-14)


def paged_case(seed, lens, page_size, Hq=24, Hkv=4, D=256, spare=3, std=1.0):
    rng = np.random.default_rng(seed)
    R = len(lens)
    need = [(L + page_size - 1) // page_size for L in lens]
    max_pages = max(need) + 1
    num_pages = sum(need) + spare
    perm = rng.permutation(num_pages)
    bt = np.full((R, max_pages), -1, np.int64)
    at = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[at:at + n]
        at += n
    rb = oracle.round_bf16
    return dict(q=rng.standard_normal((R, Hq, D)) * std, k=rng.standard_normal((R, Hkv, D)) * std,
                v=rb(rng.standard_normal((R, Hkv, D))), gate=rng.standard_normal((R, Hq, D)),
                kc=rb(rng.standard_normal((num_pages, Hkv, page_size, D))),
                vc=rb(rng.standard_normal((num_pages, Hkv, page_size, D))),
                bt=bt, lens=np.array(lens), P=page_size)


def run(c, **kw):
    return oracle.gqa_decode_paged(c["q"], c["k"], c["v"], c["gate"], c["kc"], c["vc"], c["bt"],
                                   c["lens"], c["P"], RD, THETA, **kw)


def test_attention_matches_dense_softmax():
    c = paged_case(3, [1, 5, 16, 17, 40], page_size=4)
    y, o, kc, vc = run(c)
    G = 6
    for r, L in enumerate(c["lens"]):
        # dense, contiguous keys: gather positions by hand, then put the new token last
        rows = [(c["bt"][r, j // 4], j % 4) for j in range(L - 1)]
        pos = L - 1
        qr = oracle.rope_partial(c["q"][r:r + 1], [pos], RD, THETA)[0]
        kr = oracle.round_bf16(oracle.rope_partial(c["k"][r:r + 1], [pos], RD, THETA)[0])
        for h in range(24):
            g = h // G
            K = np.array([c["kc"][p, g, off] for p, off in rows] + [kr[g]])
            V = np.array([c["vc"][p, g, off] for p, off in rows] + [c["v"][r, g]])
            w = softmax(K @ qr[h] / 16.0)
            np.testing.assert_allclose(o[r, h], w @ V, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(y[r, h], (w @ V) * expit(c["gate"][r, h]), rtol=1e-12, atol=1e-12)


def test_single_position_and_equal_keys():
    c = paged_case(4, [1, 9], page_size=8)
    y, o, _, _ = run(c)
    for h in range(24):
        np.testing.assert_allclose(o[0, h], c["v"][0, h // 6], rtol=0, atol=1e-15)   # L = 1: o = v
    # equal keys everywhere (a zero query makes every score 0): o = mean of the values
    c2 = dict(c, q=np.zeros_like(c["q"]))
    _, o2, _, vc2 = run(c2)
    for h in range(24):
        g = h // 6
        vals = [vc2[c["bt"][1, j // 8], g, j % 8] for j in range(9)]
        np.testing.assert_allclose(o2[1, h], np.mean(vals, axis=0), rtol=0, atol=1e-14)


def test_zero_gate_halves_and_large_gate_passes():
    c = paged_case(5, [3, 6], page_size=2)
    c0 = dict(c, gate=np.zeros_like(c["gate"]))
    y, o, _, _ = run(c0)
    np.testing.assert_array_equal(y, o / 2)
    cb = dict(c, gate=np.full_like(c["gate"], 50.0))
    y, o, _, _ = run(cb)
    np.testing.assert_allclose(y, o, rtol=1e-20, atol=1e-20)


def test_append_writes_only_the_new_position():
    c = paged_case(6, [7, 12, 1], page_size=4)
    _, _, kc, vc = run(c)
    changed = set()
    for r, L in enumerate(c["lens"]):
        p, off = c["bt"][r, (L - 1) // 4], (L - 1) % 4
        kr = oracle.rope_partial(c["k"][r:r + 1], [L - 1], RD, THETA)[0]
        np.testing.assert_array_equal(kc[p, :, off], oracle.round_bf16(kr))
        np.testing.assert_array_equal(vc[p, :, off], c["v"][r])
        changed.add((p, off))
    mask = np.ones(kc.shape[:1] + kc.shape[2:3], bool)
    for p, off in changed:
        mask[p, off] = False
    np.testing.assert_array_equal(kc.transpose(0, 2, 1, 3)[mask], c["kc"].transpose(0, 2, 1, 3)[mask])
    np.testing.assert_array_equal(vc.transpose(0, 2, 1, 3)[mask], c["vc"].transpose(0, 2, 1, 3)[mask])


def test_page_relocation_and_garbage_beyond_length():
    """Moving every page to another physical id (and its table entries with it)
    changes nothing; neither do cache entries past a request's length."""
    c = paged_case(7, [10, 3, 21], page_size=4, spare=5)
    y, o, kc, vc = run(c)
    rng = np.random.default_rng(70)
    perm = rng.permutation(c["kc"].shape[0])           # old page p -> new page perm[p]
    kc2 = np.empty_like(c["kc"])
    vc2 = np.empty_like(c["vc"])
    kc2[perm] = c["kc"]
    vc2[perm] = c["vc"]
    bt2 = np.where(c["bt"] >= 0, perm[np.maximum(c["bt"], 0)], -1)
    c2 = dict(c, kc=kc2, vc=vc2, bt=bt2)
    y2, o2, _, _ = run(c2)
    np.testing.assert_array_equal(o2, o)
    # garbage past each length (the rest of the last page, unused pages)
    c3 = dict(c, kc=c["kc"].copy(), vc=c["vc"].copy())
    used = set()
    for r, L in enumerate(c["lens"]):
        for j in range(L):
            used.add((c["bt"][r, j // 4], j % 4))
    for p in range(c3["kc"].shape[0]):
        for off in range(4):
            if (p, off) not in used:
                c3["kc"][p, :, off] = 1e3
                c3["vc"][p, :, off] = -1e3
    _, o3, _, _ = run(c3)
    np.testing.assert_array_equal(o3, o)


def test_head_sharing_query_7_reads_kv_1():
    c = paged_case(8, [6, 6], page_size=8)
    _, o, _, _ = run(c)
    c2 = dict(c, kc=c["kc"].copy(), vc=c["vc"].copy(), k=c["k"].copy(), v=c["v"].copy())
    c2["kc"][:, 1] = oracle.round_bf16(np.random.default_rng(80).standard_normal(c2["kc"][:, 1].shape))
    c2["vc"][:, 1] *= -1
    c2["k"][:, 1] *= 2
    c2["v"][:, 1] *= -1
    _, o2, _, _ = run(c2)
    changed = [h for h in range(24) if not np.array_equal(o2[:, h], o[:, h])]
    assert changed == list(range(6, 12))     # query heads 6 .. 11 (7 among them) read kv head 1


def test_contract_errors():
    c = paged_case(9, [5, 8], page_size=4)
    with pytest.raises(ValueError):
        _check_paged(c["bt"], np.array([0, 8]), 4, c["kc"].shape[0])         # empty context
    with pytest.raises(ValueError):
        _check_paged(c["bt"], np.array([5, 100]), 4, c["kc"].shape[0])       # beyond the table
    bad = c["bt"].copy()
    bad[1, 1] = bad[0, 1]        # request 1 reads the page request 0 appends to
    with pytest.raises(ValueError):
        _check_paged(bad, c["lens"], 4, c["kc"].shape[0])
    bad = c["bt"].copy()
    bad[0, 0] = c["kc"].shape[0]
    with pytest.raises(ValueError):
        _check_paged(bad, c["lens"], 4, c["kc"].shape[0])


# ---------------------------------------------------------------- fp8 e4m3 cache

def test_e4m3_decode_matches_torch_float8():
    import torch
    got = oracle.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9        # largest normal, smallest subnormal


def test_e4m3_round_matches_torch_and_ties_to_even():
    import torch
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200000) * np.exp2(rng.uniform(-14, 9, 200000))).astype(np.float32).astype(np.float64)
    x = x[np.abs(x) < 440]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_round(x), ref)
    # halfway cases go to the even mantissa; saturation at +-448
    cases = {1 + 1 / 16: 1.0, 1 + 3 / 16: 1.25, 2.0 ** -10: 0.0, 1.5 * 2.0 ** -9: 2.0 ** -8,
             -(1 + 1 / 16): -1.0, 464.0: 448.0, 500.0: 448.0, -1e9: -448.0, 0.0: 0.0}
    for a, b in cases.items():
        assert oracle.e4m3_round(a) == b, (a, oracle.e4m3_round(a), b)
    # every finite code round-trips
    vals = oracle.e4m3_decode(np.arange(256))
    fin = ~np.isnan(vals)
    codes = oracle.e4m3_encode(vals[fin])
    np.testing.assert_array_equal(codes, np.arange(256)[fin].astype(np.uint8))


def test_fp8_cache_append_and_attention():
    c = paged_case(12, [1, 9, 33], page_size=8)
    ks, vs = 0.5, 2.0
    kc = ks * oracle.e4m3_round(c["kc"] / ks)
    vc = vs * oracle.e4m3_round(c["vc"] / vs)
    y, o, kc2, vc2 = oracle.gqa_decode_paged(c["q"], c["k"], c["v"], c["gate"], kc, vc, c["bt"], c["lens"],
                                             c["P"], RD, THETA, cache_round=oracle.fp8_cache_round(ks),
                                             v_round=oracle.fp8_cache_round(vs))
    for r, L in enumerate(c["lens"]):
        p, off = c["bt"][r, (L - 1) // 8], (L - 1) % 8
        kr = oracle.rope_partial(c["k"][r:r + 1], [L - 1], RD, THETA)[0]
        np.testing.assert_array_equal(kc2[p, :, off], ks * oracle.e4m3_round(kr / ks))
        np.testing.assert_array_equal(vc2[p, :, off], vs * oracle.e4m3_round(c["v"][r] / vs))
        rows = [(c["bt"][r, j // 8], j % 8) for j in range(L)]
        qr = oracle.rope_partial(c["q"][r:r + 1], [L - 1], RD, THETA)[0]
        for h in (0, 7, 23):
            K = np.array([kc2[pp, h // 6, oo] for pp, oo in rows])
            V = np.array([vc2[pp, h // 6, oo] for pp, oo in rows])
            np.testing.assert_allclose(o[r, h], softmax(K @ qr[h] / 16.0) @ V, rtol=1e-12, atol=1e-12)
    # every stored value is a scaled e4m3 value
    assert np.all(oracle.e4m3_round(kc2 / ks) == kc2 / ks)
