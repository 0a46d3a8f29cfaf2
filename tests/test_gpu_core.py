"""GPU parity of the conv, decode, gated-norm and prefill entry points against
the fp64 oracle, called through the C ABI on seeded inputs.

Per-call parity feeds each oracle stage the exact values the GPU stage
received; chained runs feed the oracle the original inputs and compare the
end of the chain.  Conv history and slot placement are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import FP32_TOL, OUT_TOL, STATE_TOL, bf16_ulp_ok, bits, check_y_rows, dev, f64, rel_l2
from hybrid_linear_attention_amd import gdn
from hybrid_linear_attention_amd.workloads import (FULL_DIMS, TINY_DIMS, GdnDims, decode_r64,
                                                   make_gdn_case, tiny_core)

pytestmark = pytest.mark.gpu

L2_EPS = 1e-6
NORM_EPS = 1e-6


def dims_t(d):
    return (d.num_k_heads, d.num_v_heads, d.head_dim_k, d.head_dim_v, d.conv_taps)


def run_conv_gpu(case, act_dtype=torch.float32):
    d = case.dims
    T = case.num_tokens
    q = torch.empty((T, d.num_k_heads, d.head_dim_k), dtype=act_dtype, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((T, d.num_v_heads, d.head_dim_v), dtype=act_dtype, device="cuda")
    pool = dev(case.conv_pool)
    gdn.gdn_conv1d_update(d, dev(case.x_qkv), dev(case.conv_w), pool, dev(case.qsl),
                          dev(case.slot_ids), dev(case.has_initial), q, k, v, l2_eps=L2_EPS)
    return q, k, v, pool


def oracle_conv(case):
    d = case.dims
    return oracle.conv1d_update(f64(case.x_qkv), f64(case.conv_w), f64(case.conv_pool),
                                case.qsl.numpy(), case.slot_ids.numpy(), case.has_initial.numpy(),
                                d.num_k_heads, d.num_v_heads, d.head_dim_k, d.head_dim_v, L2_EPS)


def check_pool(case, got_pool, ref_pool):
    """Used slots: bit-exact against the oracle's history; unused: bits unchanged."""
    gb = bits(got_pool)
    ib = bits(case.conv_pool)
    used = set(int(s) for s in case.slot_ids)
    for s in range(case.num_slots):
        if s in used:
            ref = torch.from_numpy(ref_pool[s]).to(case.conv_pool.dtype)
            np.testing.assert_array_equal(gb[s], bits(ref), err_msg=f"history slot {s}")
        else:
            np.testing.assert_array_equal(gb[s], ib[s], err_msg=f"unused slot {s} touched")


def varlen_case(seed, D=128, Hk=2, Hv=6, lengths=(1, 2, 5, 37, 0, 130, 3), num_slots=10,
                dtype=torch.bfloat16, state_std=0.02, hist_std=1.0, mixed_init=True):
    c = make_gdn_case(seed, GdnDims(Hk, Hv, D, D, 4), list(lengths), num_slots=num_slots,
                      permute_slots=True, act_dtype=dtype, state_std=state_std,
                      hist_std=hist_std)
    if mixed_init:
        c.has_initial = torch.tensor([(r % 3) != 1 for r in range(c.num_reqs)], dtype=torch.uint8)
    return c


# ---------------------------------------------------------------------------
# conv1d + SiLU + L2 norm
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("which", ["tiny", "varlen_bf16", "varlen_f32_d16", "decode_r64"])
def test_conv_parity(which):
    if which == "tiny":
        case = tiny_core()
    elif which == "varlen_bf16":
        case = varlen_case(11)
    elif which == "varlen_f32_d16":
        case = varlen_case(12, D=16, Hk=3, Hv=6, dtype=torch.float32)
    else:
        case = decode_r64()
    q, k, v, pool = run_conv_gpu(case)
    qr, kr, vr, pr = oracle_conv(case)
    for name, got, ref in (("q", q, qr), ("k", k, kr), ("v", v, vr)):
        err = rel_l2(f64(got), ref)
        assert err <= FP32_TOL, f"{which} {name} rel-L2 {err:.3e}"
    check_pool(case, pool, pr)


def test_conv_bf16_outputs_round_once():
    case = varlen_case(13)
    q, k, v, _ = run_conv_gpu(case, act_dtype=torch.bfloat16)
    qr, kr, vr, _ = oracle_conv(case)
    for got, ref in ((q, qr), (k, kr), (v, vr)):
        assert bf16_ulp_ok(got, ref, ulps=1)


def test_conv_strided_input_rows():
    """x as a column slice of a wider row (the in-projection's q|k|v|z output)."""
    case = varlen_case(14, lengths=(3, 9, 1))
    d = case.dims
    C = d.conv_channels
    wide = torch.randn(case.num_tokens, C + 40, dtype=case.x_qkv.dtype)
    wide[:, :C] = case.x_qkv
    T = case.num_tokens
    q = torch.empty((T, d.num_k_heads, d.head_dim_k), device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((T, d.num_v_heads, d.head_dim_v), device="cuda")
    pool = dev(case.conv_pool)
    gdn.gdn_conv1d_update(d, dev(wide)[:, :C], dev(case.conv_w), pool, dev(case.qsl),
                          dev(case.slot_ids), dev(case.has_initial), q, k, v, l2_eps=L2_EPS)
    qr, kr, vr, pr = oracle_conv(case)
    assert rel_l2(f64(v), vr) <= FP32_TOL and rel_l2(f64(q), qr) <= FP32_TOL
    check_pool(case, pool, pr)


def long_lengths(seed, n, hi):
    """Request lengths for batches above 1024 tokens (the vectorised conv path):
    many 0-3 token requests mixed with longer ones, so request starts fall at
    every offset of a token tile."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(0, hi, n)]
    lens[::5] = [int(x) for x in rng.integers(0, 4, len(lens[::5]))]
    lens += [1100 - sum(lens)] if sum(lens) < 1100 else []
    return lens


@pytest.mark.parametrize("which", ["d128_bf16", "d16_f32", "d64_bf16_out", "d32_tile_edges"])
def test_conv_long_batch_parity(which):
    if which == "d128_bf16":
        case = varlen_case(21, lengths=long_lengths(21, 40, 80), num_slots=48)
        act = torch.float32
    elif which == "d16_f32":
        case = varlen_case(22, D=16, Hk=3, Hv=6, dtype=torch.float32,
                           lengths=long_lengths(22, 90, 40), num_slots=100)
        act = torch.float32
    elif which == "d64_bf16_out":
        case = varlen_case(23, D=64, Hk=2, Hv=4, lengths=long_lengths(23, 60, 50), num_slots=64)
        act = torch.bfloat16
    else:
        # requests of 15, 16, 17 tokens and 1-3 token requests straddling tile ends
        lens = [1, 2, 0, 15, 16, 17, 3, 33, 1, 1, 2, 14, 0, 46, 31, 2, 3, 13, 1, 18] * 4
        case = varlen_case(24, D=32, Hk=2, Hv=4, lengths=lens + [1200], num_slots=90)
        act = torch.float32
    assert case.num_tokens > 1024
    q, k, v, pool = run_conv_gpu(case, act_dtype=act)
    qr, kr, vr, pr = oracle_conv(case)
    for name, got, ref in (("q", q, qr), ("k", k, kr), ("v", v, vr)):
        if act == torch.bfloat16:
            assert bf16_ulp_ok(got, ref, ulps=1), f"{which} {name}"
        else:
            err = rel_l2(f64(got), ref)
            assert err <= FP32_TOL, f"{which} {name} rel-L2 {err:.3e}"
    check_pool(case, pool, pr)


@pytest.mark.parametrize("extra", [40, 37])
def test_conv_long_batch_strided(extra):
    """x as a column slice of a wider row at more than 1024 tokens: a row stride
    of 1320 bf16 (16-byte rows) takes the vectorised kernel, a stride of 1318
    (even, but rows not 16-byte aligned) the per-token kernel; both must match."""
    case = varlen_case(25, lengths=long_lengths(25, 30, 90), num_slots=40)
    d = case.dims
    C = d.conv_channels
    width = C + extra + (extra % 2)  # the ABI needs an even stride
    wide = torch.randn(case.num_tokens, width, dtype=case.x_qkv.dtype)
    wide[:, :C] = case.x_qkv
    T = case.num_tokens
    q = torch.empty((T, d.num_k_heads, d.head_dim_k), device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((T, d.num_v_heads, d.head_dim_v), device="cuda")
    pool = dev(case.conv_pool)
    gdn.gdn_conv1d_update(d, dev(wide)[:, :C], dev(case.conv_w), pool, dev(case.qsl),
                          dev(case.slot_ids), dev(case.has_initial), q, k, v, l2_eps=L2_EPS)
    qr, kr, vr, pr = oracle_conv(case)
    for got, ref in ((q, qr), (k, kr), (v, vr)):
        assert rel_l2(f64(got), ref) <= FP32_TOL
    check_pool(case, pool, pr)


# ---------------------------------------------------------------------------
# decode step
# ---------------------------------------------------------------------------
def run_decode_gpu(d, q, k, v, a, b, state_pool, slot_ids, o_dtype=torch.float32):
    o = torch.empty((q.shape[0], d.num_v_heads, d.head_dim_v), dtype=o_dtype, device="cuda")
    gdn.gdn_decode_step(d, q, k, v, a, b, state_pool, slot_ids, o)
    return o


@pytest.mark.parametrize("D,Hk,Hv,R,nslots", [(128, 16, 48, 64, 64), (128, 2, 6, 5, 9),
                                              (16, 2, 6, 7, 7), (32, 1, 2, 3, 8),
                                              (64, 4, 4, 33, 40)])
def test_decode_step_parity(D, Hk, Hv, R, nslots):
    """Per-call parity: the oracle gets the exact q/k/v/a/b the kernel got."""
    rng = np.random.default_rng(D * 1000 + R)
    d = GdnDims(Hk, Hv, D, D, 4)
    q = torch.from_numpy(oracle.l2norm(rng.standard_normal((R, Hk, D)), 0)).float()
    k = torch.from_numpy(oracle.l2norm(rng.standard_normal((R, Hk, D)), 0)).float()
    v = torch.from_numpy(rng.standard_normal((R, Hv, D))).float()
    a = torch.from_numpy(rng.standard_normal((R, Hv))).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal((R, Hv))).to(torch.bfloat16)
    pool = torch.from_numpy(rng.standard_normal((nslots, Hv, D, D)) * 0.02).float()
    slots = torch.from_numpy(rng.permutation(nslots)[:R].astype(np.int32))
    gpool = dev(pool)
    o = run_decode_gpu(d, dev(q), dev(k), dev(v), dev(a), dev(b), gpool, dev(slots))
    o_ref, pool_ref = oracle.decode_step(f64(q), f64(k), f64(v), f64(a), f64(b), f64(pool),
                                         slots.numpy())
    assert rel_l2(f64(o), o_ref) <= 1e-5
    assert rel_l2(f64(gpool), pool_ref) <= 1e-6
    unused = sorted(set(range(nslots)) - set(slots.tolist()))
    if unused:
        np.testing.assert_array_equal(bits(gpool)[unused], bits(pool)[unused])


def test_decode_bf16_inputs_and_output():
    rng = np.random.default_rng(5)
    R, Hk, Hv, D = 8, 2, 6, 128
    d = GdnDims(Hk, Hv, D, D, 4)
    q = torch.from_numpy(oracle.l2norm(rng.standard_normal((R, Hk, D)), 0)).to(torch.bfloat16)
    k = torch.from_numpy(oracle.l2norm(rng.standard_normal((R, Hk, D)), 0)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((R, Hv, D))).to(torch.bfloat16)
    ab = torch.from_numpy(rng.standard_normal((R, 2 * Hv + 4))).float()
    a, b = ab[:, :Hv], ab[:, Hv:2 * Hv]  # strided gate views (gate_ld = 2*Hv + 4)
    pool = torch.from_numpy(rng.standard_normal((R, Hv, D, D)) * 0.02).float()
    slots = torch.arange(R, dtype=torch.int32)
    gab = dev(ab)
    gpool = dev(pool)
    o = run_decode_gpu(d, dev(q), dev(k), dev(v), gab[:, :Hv], gab[:, Hv:2 * Hv], gpool,
                       dev(slots), o_dtype=torch.bfloat16)
    o_ref, pool_ref = oracle.decode_step(f64(q), f64(k), f64(v), f64(a), f64(b), f64(pool),
                                         slots.numpy())
    assert bf16_ulp_ok(o, o_ref, ulps=1)
    assert rel_l2(f64(gpool), pool_ref) <= 1e-6


def test_decode_chain_full_size():
    """Full-size decode step as a chain: conv1d_update -> decode_step -> gated_norm
    on 64 requests x 48 value heads, against the oracle fed the original inputs."""
    case = decode_r64()
    d = case.dims
    q, k, v, pool = run_conv_gpu(case)
    state = dev(case.state_pool)
    o = run_decode_gpu(d, q, k, v, dev(case.a), dev(case.b), state, dev(case.slot_ids))
    y = torch.empty((case.num_tokens, d.num_v_heads * d.head_dim_v), dtype=torch.bfloat16,
                    device="cuda")
    gdn.gdn_gated_norm(d, o, dev(case.z), dev(case.gamma), y, eps=NORM_EPS)
    qr, kr, vr, pr = oracle_conv(case)
    o_ref, st_ref = oracle.decode_step(qr, kr, vr, f64(case.a), f64(case.b), f64(case.state_pool),
                                       case.slot_ids.numpy())
    y_ref = oracle.gated_norm(o_ref, f64(case.z), f64(case.gamma), NORM_EPS)
    e_o, e_s, e_y = rel_l2(f64(o), o_ref), rel_l2(f64(state), st_ref), rel_l2(f64(y), y_ref)
    print(f"decode chain rel-L2: o {e_o:.2e} state {e_s:.2e} y {e_y:.2e}")
    assert e_o <= OUT_TOL and e_s <= STATE_TOL and e_y <= OUT_TOL
    check_pool(case, pool, pr)


def run_fused_gpu(case, y_dtype=torch.bfloat16, x=None, z=None, a=None, b=None):
    d = case.dims
    R = case.num_reqs
    pool = dev(case.conv_pool)
    state = dev(case.state_pool)
    y = torch.empty((R, d.num_v_heads * d.head_dim_v), dtype=y_dtype, device="cuda")
    o = torch.empty((R, d.num_v_heads, d.head_dim_v), device="cuda")
    gdn.gdn_decode_fused(d, dev(case.x_qkv) if x is None else x, dev(case.z) if z is None else z,
                         dev(case.a) if a is None else a, dev(case.b) if b is None else b,
                         dev(case.conv_w), dev(case.gamma), pool, state, dev(case.slot_ids), y,
                         has_initial=dev(case.has_initial), o=o, l2_eps=L2_EPS,
                         norm_eps=NORM_EPS)
    return y, o, pool, state


def oracle_decode_chain(case):
    """conv update -> one recurrence step per request (zero state where
    has_initial is 0) -> gated norm, in fp64 on the exact inputs."""
    d = case.dims
    qr, kr, vr, pr = oracle_conv(case)
    o_ref, st_ref = oracle.gated_delta_rule(qr, kr, vr, f64(case.a), f64(case.b),
                                            f64(case.state_pool), case.qsl.numpy(),
                                            case.slot_ids.numpy(), case.has_initial.numpy())
    z = f64(case.z).reshape(case.num_tokens, d.num_v_heads, d.head_dim_v)
    y_ref = oracle.gated_norm(o_ref, z, f64(case.gamma), NORM_EPS)
    return o_ref, y_ref, st_ref, pr


def check_state_slots(case, got, ref, tol):
    used = sorted(set(int(s) for s in case.slot_ids))
    e = rel_l2(f64(got)[used], ref[used])
    unused = sorted(set(range(case.num_slots)) - set(used))
    if unused:
        np.testing.assert_array_equal(bits(got)[unused], bits(case.state_pool)[unused])
    return e


def fused_case(which):
    if which == "decode_r64":
        return decode_r64(), torch.bfloat16
    if which == "d32_g2":
        # d = 32 (4 lanes a state row), 2 value heads per key head, bf16
        return make_gdn_case(33, GdnDims(3, 6, 32, 32, 4), [1] * 13, num_slots=20, permute_slots=True,
                             state_std=0.02, hist_std=1.0, gamma_std=0.1), torch.bfloat16
    if which == "tiny_f32":
        c = make_gdn_case(31, TINY_DIMS, [1] * 9, num_slots=14, permute_slots=True,
                          act_dtype=torch.float32, state_std=0.02, hist_std=1.0, gamma_std=0.1)
        c.has_initial = torch.tensor([r % 4 != 2 for r in range(9)], dtype=torch.uint8)
        return c, torch.float32
    c = make_gdn_case(32, GdnDims(2, 8, 64, 64, 4), [1] * 21, num_slots=30, permute_slots=True,
                      state_std=0.02, hist_std=1.0, gamma_std=0.1)
    return c, torch.bfloat16


@pytest.mark.parametrize("which", ["decode_r64", "tiny_f32", "d64_g4", "d32_g2"])
def test_decode_fused_parity(which):
    """One-launch decode step against the fp64 oracle chain: o (fp32 copy) and
    states to fp32 accuracy, y within one rounding, history bit-exact, unused
    slots untouched."""
    case, ydt = fused_case(which)
    y, o, pool, state = run_fused_gpu(case, y_dtype=ydt)
    o_ref, y_ref, st_ref, pr = oracle_decode_chain(case)
    e_o = rel_l2(f64(o), o_ref)
    e_s = check_state_slots(case, state, st_ref, FP32_TOL)
    print(f"{which}: o {e_o:.2e} state {e_s:.2e}")
    assert e_o <= FP32_TOL and e_s <= FP32_TOL
    y_ref = y_ref.reshape(case.num_tokens, -1)
    if ydt == torch.bfloat16:
        assert bf16_ulp_ok(y, y_ref, ulps=1)
    else:
        assert rel_l2(f64(y), y_ref) <= FP32_TOL
    check_pool(case, pool, pr)


def test_decode_fused_matches_three_calls_strided():
    """x, z, a and b as column slices of one wide projection row (the layer's
    layout): the fused step equals conv1d_update -> decode_step -> gated_norm."""
    case, _ = fused_case("d64_g4")
    d = case.dims
    R = case.num_reqs
    C = d.conv_channels
    Hv, D = d.num_v_heads, d.head_dim_v
    width = C + Hv * D + 2 * Hv + 8
    wide = torch.zeros((R, width), dtype=torch.bfloat16)
    wide[:, :C] = case.x_qkv
    wide[:, C:C + Hv * D] = case.z.reshape(R, -1)
    wide[:, C + Hv * D:C + Hv * D + Hv] = case.b
    wide[:, C + Hv * D + Hv:C + Hv * D + 2 * Hv] = case.a
    W = dev(wide)
    xs, zs = W[:, :C], W[:, C:C + Hv * D]
    bs, as_ = W[:, C + Hv * D:C + Hv * D + Hv], W[:, C + Hv * D + Hv:C + Hv * D + 2 * Hv]
    y1, o1, pool1, state1 = run_fused_gpu(case, x=xs, z=zs, a=as_, b=bs)
    # the three separate entry points on the same views
    pool2, state2 = dev(case.conv_pool), dev(case.state_pool)
    q = torch.empty((R, d.num_k_heads, d.head_dim_k), device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((R, Hv, D), device="cuda")
    gdn.gdn_conv1d_update(d, xs, dev(case.conv_w), pool2, dev(case.qsl), dev(case.slot_ids),
                          dev(case.has_initial), q, k, v, l2_eps=L2_EPS)
    o2 = run_decode_gpu(d, q, k, v, as_, bs, state2, dev(case.slot_ids))
    y2 = torch.empty((R, Hv * D), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_gated_norm(d, o2, zs, dev(case.gamma), y2, eps=NORM_EPS)
    np.testing.assert_array_equal(bits(pool1), bits(pool2))
    used = sorted(set(int(s) for s in case.slot_ids))
    unused = sorted(set(range(case.num_slots)) - set(used))
    assert rel_l2(f64(state1)[used], f64(state2)[used]) <= 1e-6
    np.testing.assert_array_equal(bits(state1)[unused], bits(state2)[unused])
    assert rel_l2(f64(o1), f64(o2)) <= 1e-6
    assert bf16_ulp_ok(y1, f64(y2), ulps=1)


def test_tiny_core_as_decode_steps():
    """The tiny workload (T=64, fp32) run as 64 single-token steps (conv then decode)
    against the oracle's whole-sequence result."""
    case = tiny_core()
    d = case.dims
    pool = dev(case.conv_pool)
    state = dev(case.state_pool)
    x = dev(case.x_qkv)
    a, b = dev(case.a), dev(case.b)
    qsl1 = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    slot = torch.zeros(1, dtype=torch.int32, device="cuda")
    hi = torch.ones(1, dtype=torch.uint8, device="cuda")
    outs = []
    for t in range(case.num_tokens):
        q = torch.empty((1, d.num_k_heads, d.head_dim_k), device="cuda")
        k = torch.empty_like(q)
        v = torch.empty((1, d.num_v_heads, d.head_dim_v), device="cuda")
        gdn.gdn_conv1d_update(d, x[t:t + 1], dev(case.conv_w), pool, qsl1, slot, hi, q, k, v,
                              l2_eps=L2_EPS)
        outs.append(run_decode_gpu(d, q, k, v, a[t:t + 1], b[t:t + 1], state, slot))
    o = torch.cat(outs)
    qr, kr, vr, pr = oracle_conv(case)
    o_ref, st_ref = oracle.gated_delta_rule(qr, kr, vr, f64(case.a), f64(case.b),
                                            f64(case.state_pool), case.qsl.numpy(),
                                            case.slot_ids.numpy(), case.has_initial.numpy())
    assert rel_l2(f64(o), o_ref) <= 1e-5
    assert rel_l2(f64(state), st_ref) <= 1e-5
    check_pool(case, pool, pr)


# ---------------------------------------------------------------------------
# gated RMSNorm
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D,Hv,T,odt,ydt,zoff", [(128, 48, 37, torch.float32, torch.bfloat16, 8),
                                                 (16, 6, 64, torch.float32, torch.float32, 8),
                                                 (64, 5, 3, torch.bfloat16, torch.float32, 8),
                                                 (128, 48, 37, torch.float32, torch.bfloat16, 2),
                                                 (32, 6, 50, torch.float32, torch.float32, 6),
                                                 (128, 48, 6000, torch.float32, torch.bfloat16, 8),
                                                 (64, 8, 33000, torch.bfloat16, torch.float32, 8)])
def test_gated_norm_parity(D, Hv, T, odt, ydt, zoff):
    """z is a column slice of a wider row (z_ld = Hv*D + 16): a slice starting 8
    columns in keeps 16-byte rows (vectorised kernel; the two large cases use
    several rows per thread), an offset of 2 or 6 does not (per-pair kernel)."""
    rng = np.random.default_rng(D + T)
    d = GdnDims(1, Hv, D, D, 4)
    o = torch.from_numpy(rng.standard_normal((T, Hv, D)) * rng.uniform(0.01, 3, (T, Hv, 1))).to(odt)
    zw = torch.from_numpy(rng.standard_normal((T, Hv * D + 16))).to(torch.bfloat16)
    z = zw[:, zoff:zoff + Hv * D]
    g = torch.from_numpy(1 + 0.1 * rng.standard_normal(D)).to(torch.bfloat16)
    y = torch.empty((T, Hv * D), dtype=ydt, device="cuda")
    gdn.gdn_gated_norm(d, dev(o), dev(zw)[:, zoff:zoff + Hv * D], dev(g), y, eps=NORM_EPS)
    y_ref = oracle.gated_norm(f64(o), f64(z).reshape(T, Hv, D), f64(g), NORM_EPS)
    if ydt == torch.bfloat16:
        assert bf16_ulp_ok(y, y_ref, ulps=1)
    else:
        assert rel_l2(f64(y), y_ref) <= FP32_TOL


# ---------------------------------------------------------------------------
# fused prefill step (conv update -> recurrence -> gated norm)
# ---------------------------------------------------------------------------
def run_prefill_fused_gpu(case, y_dtype=torch.bfloat16, x_pad=0):
    """x_pad > 0 passes x as a column slice of rows x_pad elements wider."""
    d = case.dims
    T = case.num_tokens
    pool = dev(case.conv_pool)
    state = dev(case.state_pool)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=y_dtype, device="cuda")
    nbytes = gdn.gdn_prefill_fused_workspace_bytes(d, T, case.num_reqs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x = dev(case.x_qkv)
    if x_pad:
        C = d.conv_channels
        wide = torch.zeros((T, C + x_pad), dtype=case.x_qkv.dtype, device="cuda")
        wide[:, :C] = x
        x = wide[:, :C]
    gdn.gdn_prefill_fused(d, x, dev(case.z), dev(case.a), dev(case.b),
                          dev(case.conv_w), dev(case.gamma), pool, state, dev(case.qsl),
                          dev(case.slot_ids), dev(case.has_initial), y, ws, l2_eps=L2_EPS,
                          norm_eps=NORM_EPS)
    return y, pool, state


@pytest.mark.parametrize("which", ["d128_split_rows", "d128_whole_heads", "d128_group_f32y", "d32_seq",
                                   "d64_seq", "d128_unaligned_rows", "d128_many_requests", "d128_f32x_rows",
                                   "d128_f32x_heads"])
def test_prefill_fused_parity(which):
    """One prefill step through gdn_prefill_fused against the fp64 oracle chain:
    32-row chain blocks (few heads x requests); whole-head blocks that form the
    gated output themselves (>= 256 (request, head) units, bf16 y); key-head
    group blocks with the separate gated-norm pass (the same units, fp32 y); the
    sequential kernel for d = 32; x rows that are not 16-byte aligned (the
    conv pass then forms q and k before the prep kernel instead of the prep
    kernel forming them from x); and fp32 activations (the prep kernel convolves
    the q and k channels in two passes), with few units and with >= 256."""
    x_pad = 0
    y_dtype = torch.bfloat16
    if which == "d128_split_rows":
        case = varlen_case(41, lengths=(1, 2, 5, 37, 0, 130, 3), num_slots=10)
    elif which == "d128_unaligned_rows":
        case = varlen_case(44, lengths=(3, 50, 0, 2, 91), num_slots=7)
        x_pad = 2
    elif which in ("d128_whole_heads", "d128_group_f32y"):
        rng = np.random.default_rng(42)
        lens = [int(x) for x in rng.integers(0, 70, 48)]
        case = varlen_case(42, lengths=lens, num_slots=60)
        if which == "d128_group_f32y":
            y_dtype = torch.float32
    elif which == "d128_f32x_rows":
        case = varlen_case(46, lengths=(1, 2, 5, 37, 0, 130, 3), num_slots=10, dtype=torch.float32)
        y_dtype = torch.float32
    elif which == "d128_f32x_heads":
        rng = np.random.default_rng(47)
        lens = [int(x) for x in rng.integers(0, 70, 48)]
        case = varlen_case(47, lengths=lens, num_slots=60, dtype=torch.float32)
        y_dtype = torch.float32
    elif which == "d128_many_requests":
        # more than 64 requests: the chunk plan comes from the plan kernel
        rng = np.random.default_rng(45)
        lens = [int(x) for x in rng.integers(0, 70, 100)]
        case = varlen_case(45, lengths=lens, num_slots=104)
    elif which == "d64_seq":
        case = varlen_case(48, D=64, Hk=2, Hv=8, lengths=(5, 66, 0, 31, 2), num_slots=7)
    else:
        case = varlen_case(43, D=32, Hk=2, Hv=4, lengths=(3, 40, 1, 77), num_slots=6)
    y, pool, state = run_prefill_fused_gpu(case, y_dtype=y_dtype, x_pad=x_pad)
    d = case.dims
    qr, kr, vr, pr = oracle_conv(case)
    o_ref, st_ref = oracle.gated_delta_rule(qr, kr, vr, f64(case.a), f64(case.b),
                                            f64(case.state_pool), case.qsl.numpy(),
                                            case.slot_ids.numpy(), case.has_initial.numpy())
    z = f64(case.z).reshape(case.num_tokens, d.num_v_heads, d.head_dim_v)
    y_ref = oracle.gated_norm(o_ref, z, f64(case.gamma), NORM_EPS).reshape(case.num_tokens, -1)
    e_y = rel_l2(f64(y), y_ref)
    e_s = check_state_slots(case, state, st_ref, STATE_TOL)
    # every (token, head) row within the bound the o rows' bound implies (the
    # gated norm divides by the row's own RMS, so a row whose o nearly cancels
    # carries the contraction's absolute error; the derived bound allows for it)
    worst = check_y_rows(f64(y), y_ref, o_ref, z, f64(case.gamma), d.head_dim_v)
    print(f"{which}: y {e_y:.2e} (worst row {worst:.2f} x bound) state {e_s:.2e}")
    assert e_y <= OUT_TOL and e_s <= STATE_TOL
    check_pool(case, pool, pr)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
def run_prefill_gpu(case, q, k, v, state, o_dtype=torch.float32):
    d = case.dims
    o = torch.empty((case.num_tokens, d.num_v_heads, d.head_dim_v), dtype=o_dtype, device="cuda")
    nbytes = gdn.gdn_prefill_workspace_bytes(d, case.num_tokens, case.num_reqs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    gdn.gdn_prefill_varlen(d, q, k, v, dev(case.a), dev(case.b), state, dev(case.qsl),
                           dev(case.slot_ids), dev(case.has_initial), o, ws)
    return o


def check_states(case, got_state, ref_state, tol):
    used = [int(s) for s, L in zip(case.slot_ids, np.diff(case.qsl.numpy()))]
    touched = [int(s) for s, L in zip(case.slot_ids, np.diff(case.qsl.numpy())) if L > 0]
    g = f64(got_state)
    if touched:
        err = rel_l2(g[touched], ref_state[touched])
        assert err <= tol, f"state rel-L2 {err:.3e}"
    untouched = sorted(set(range(case.num_slots)) - set(touched))
    if untouched:
        np.testing.assert_array_equal(bits(got_state)[untouched], bits(case.state_pool)[untouched])
    return used


@pytest.mark.parametrize("which", ["tiny", "varlen_d128", "varlen_d32", "varlen_d64", "group_blocks",
                                   "whole_head_blocks", "many_requests"])
def test_prefill_chain_parity(which):
    """The prefill entry point on each chain shape: 32-row blocks (few heads x
    requests), key-head group blocks (>= 256 heads x requests, 3 value heads per
    key head), whole-head blocks (>= 256, 4 value heads per key head), and the
    sequential kernel for d = 32.  Up to 64 requests the kernels work out the
    chunk plan in-wave; many_requests (100) takes the plan kernel."""
    if which == "tiny":
        case = tiny_core()
    elif which == "varlen_d128":
        case = varlen_case(21, lengths=(1, 64, 65, 130, 0, 7, 200))
    elif which == "group_blocks":
        rng = np.random.default_rng(26)
        case = varlen_case(26, lengths=[int(x) for x in rng.integers(0, 100, 48)], num_slots=50)
    elif which == "whole_head_blocks":
        rng = np.random.default_rng(27)
        case = varlen_case(27, Hk=2, Hv=8, lengths=[int(x) for x in rng.integers(0, 100, 40)],
                           num_slots=41)
    elif which == "many_requests":
        rng = np.random.default_rng(28)
        case = varlen_case(28, lengths=[int(x) for x in rng.integers(0, 70, 100)], num_slots=104)
    elif which == "varlen_d64":
        case = varlen_case(29, D=64, Hk=2, Hv=8, lengths=(33, 1, 0, 64, 100), num_slots=7)
    else:
        case = varlen_case(22, D=32, Hk=2, Hv=4, lengths=(70, 1, 0, 129), num_slots=6)
    q, k, v, pool = run_conv_gpu(case)
    state = dev(case.state_pool)
    o = run_prefill_gpu(case, q, k, v, state)
    qr, kr, vr, pr = oracle_conv(case)
    o_ref, st_ref = oracle.gated_delta_rule(qr, kr, vr, f64(case.a), f64(case.b),
                                            f64(case.state_pool), case.qsl.numpy(),
                                            case.slot_ids.numpy(), case.has_initial.numpy())
    e_o = rel_l2(f64(o), o_ref)
    print(f"{which}: o rel-L2 {e_o:.2e}")
    assert e_o <= OUT_TOL
    check_states(case, state, st_ref, STATE_TOL)
    check_pool(case, pool, pr)


# ---------------------------------------------------------------------------
# RMSNorm and GEMM (layer-block stages)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols,ydt", [(37, 5120, torch.bfloat16), (5, 136, torch.float32),
                                           (3, 4096, torch.bfloat16), (3, 8184, torch.float32),
                                           (2, 12000, torch.bfloat16)])
def test_rmsnorm_parity(rows, cols, ydt):
    """Rows of 1, 2, 3, 4 and 8 vectors of 8 per thread (the kernel's register
    footprint is picked from the row width)."""
    rng = np.random.default_rng(cols)
    x = torch.from_numpy(rng.standard_normal((rows, cols))).to(torch.bfloat16)
    g = torch.from_numpy(1 + 0.02 * rng.standard_normal(cols)).to(torch.bfloat16)
    y = torch.empty((rows, cols), dtype=ydt, device="cuda")
    gdn.gdn_rmsnorm(dev(x), dev(g), y, eps=NORM_EPS)
    ref = oracle.rmsnorm(f64(x), f64(g), NORM_EPS)
    if ydt == torch.bfloat16:
        assert bf16_ulp_ok(y, ref, ulps=1)
    else:
        assert rel_l2(f64(y), ref) <= FP32_TOL


@pytest.mark.parametrize("M,N,K,res", [(300, 200, 5120, False), (129, 136, 264, True),
                                       (1, 8, 8, False), (256, 96, 5120, True),
                                       (513, 264, 64, True), (1000, 520, 640, False),
                                       (300, 520, 128, False), (257, 264, 192, True),
                                       (90 * 256 - 37, 600, 128, False)])
def test_gemm_parity(M, N, K, res):
    """K a multiple of 64 takes the 256 x 256 tile kernel (edges of M and N not
    multiples of 256 included; one, two and three 64-deep stages, where the
    refill two stages ahead runs past the end; 270 tiles, more than one per
    CU, the last row and column partial), other K the 128 x 128 one."""
    rng = np.random.default_rng(M + N + K)
    A = torch.from_numpy(rng.standard_normal((M, K))).to(torch.bfloat16)
    B = torch.from_numpy(rng.standard_normal((N, K)) * 0.02).to(torch.bfloat16)
    R = torch.from_numpy(rng.standard_normal((M, N))).to(torch.bfloat16) if res else None
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    gdn.gdn_gemm_bf16(dev(A), dev(B), C, residual=dev(R) if res else None)
    ref = oracle.linear(f64(A), f64(B).T)
    if res:
        ref = oracle.residual_add(f64(R), ref)
    assert rel_l2(f64(C), ref) <= FP32_TOL
    Cb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_gemm_bf16(dev(A), dev(B), Cb, residual=dev(R) if res else None)
    assert bf16_ulp_ok(Cb, ref, ulps=1)


@pytest.mark.parametrize("M,N,K,res", [(300, 200, 5120, False), (4300, 4000, 1024, True),
                                       (256, 16480, 5120, False), (16640, 5120, 6144, True)])
def test_gemm_split_tail(M, N, K, res):
    """gdn_gemm_bf16 with a workspace: the K stages of the tiles of the last,
    partly filled round (or of all tiles, when there are fewer than compute
    units) are dealt out to up to one block per compute unit and a second
    launch adds each tile's runs.  Shapes: 2 tiles over 40 blocks; 272 tiles
    (16 tail tiles with partial rows and columns, over 64 blocks); 65 tiles over
    256 blocks (runs that cross tile ends); the out-projection of the
    16,640-token layer batch (20 tail tiles over 256 blocks).  Checked against
    the fp64 oracle on every row (the large shapes: their first and their tail
    tile rows), for fp32 and bf16 C; a second call repeats the first bit for
    bit."""
    nbytes = gdn.gdn_gemm_bf16_workspace_bytes(M, N, K)
    assert nbytes > 0, "the shape should be split"
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(M + 7 * N + K)
    A = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(torch.bfloat16)
    B = torch.from_numpy(rng.standard_normal((N, K), dtype=np.float32) * 0.02).to(torch.bfloat16)
    R = torch.from_numpy(rng.standard_normal((M, N), dtype=np.float32)).to(torch.bfloat16) if res else None
    Ad, Bd = dev(A), dev(B)
    Rd = dev(R) if res else None
    last = 256 * ((M - 1) // 256)
    rows = np.arange(M) if M * N * K <= 4e9 else np.unique(np.concatenate([np.arange(256), np.arange(last, M)]))
    ref = oracle.linear(f64(A[rows]), f64(B).T)
    if res:
        ref = oracle.residual_add(f64(R[rows]), ref)
    for cdt in (torch.float32, torch.bfloat16):
        C = torch.empty((M, N), dtype=cdt, device="cuda")
        gdn.gdn_gemm_bf16(Ad, Bd, C, residual=Rd, workspace=ws)
        C2 = torch.full((M, N), float("nan"), dtype=cdt, device="cuda")
        gdn.gdn_gemm_bf16(Ad, Bd, C2, residual=Rd, workspace=ws)
        np.testing.assert_array_equal(bits(C.cpu()), bits(C2.cpu()))
        got = C.cpu()[torch.from_numpy(rows)]
        if cdt == torch.float32:
            assert rel_l2(f64(got), ref) <= FP32_TOL
        else:
            assert bf16_ulp_ok(got, ref, ulps=1)
    print(f"{M}x{N}x{K}: {nbytes >> 19} split blocks")
