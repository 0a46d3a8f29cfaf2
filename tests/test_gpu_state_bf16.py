"""GPU parity of the bf16-state variant (state_dt = GDN_BF16) of the fused entry
points against the fp64 oracle.

The state is read as bf16 (widened exactly), updated in fp32 and rounded once
to nearest-even on store.  The oracle takes the same widened input state,
updates it in fp64 and rounds with oracle.round_bf16.  Both sides round nearly
the same value, so the stored states must agree to within one bf16 ulp
everywhere, and exactly except where the exact value lies within the GPU's
arithmetic error of a rounding boundary: a fraction of about (relative
arithmetic error) / (relative half-ulp, ~2^-9), i.e. ~1e-4 for the fp32 decode
update and ~1e-3 for the bf16x3 chunked prefill; the tests allow 1e-3 and 1e-2.
Elements whose exact value nearly cancels are held to an absolute bound instead
(the arithmetic's absolute error, 1e-6 or 3e-5 of the state's rms), since there
one ulp is far below it.
Outputs o and y come from the fp32 arithmetic on the exact widened state and
keep the fp32 and bf16 bars of the fp32-state tests.  Untouched slots keep their
bits.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import FP32_TOL, OUT_TOL, bf16_ulp_ok, bits, check_bf16_state, dev, f64, rel_l2
from hybrid_linear_attention_amd import gdn
from hybrid_linear_attention_amd.workloads import (TINY_DIMS, GdnDims, decode_r64, make_gdn_case,
                                                   spec_verify_r64)

pytestmark = pytest.mark.gpu

L2_EPS = 1e-6
NORM_EPS = 1e-6


def bf16_case(case):
    case.state_pool = case.state_pool.to(torch.bfloat16)
    return case


def oracle_chain(case):
    d = case.dims
    qr, kr, vr, pr = oracle.conv1d_update(f64(case.x_qkv), f64(case.conv_w), f64(case.conv_pool),
                                          case.qsl.numpy(), case.slot_ids.numpy(),
                                          case.has_initial.numpy(), d.num_k_heads, d.num_v_heads,
                                          d.head_dim_k, d.head_dim_v, L2_EPS)
    o_ref, st_ref = oracle.gated_delta_rule(qr, kr, vr, f64(case.a), f64(case.b),
                                            f64(case.state_pool), case.qsl.numpy(),
                                            case.slot_ids.numpy(), case.has_initial.numpy())
    z = f64(case.z).reshape(case.num_tokens, d.num_v_heads, d.head_dim_v)
    y_ref = oracle.gated_norm(o_ref, z, f64(case.gamma), NORM_EPS)
    return o_ref, y_ref, st_ref, pr


def check_untouched(case, got_state, got_pool, used):
    rest = sorted(set(range(case.num_slots)) - set(used))
    if rest:
        np.testing.assert_array_equal(bits(got_state)[rest], bits(case.state_pool)[rest])
        np.testing.assert_array_equal(bits(got_pool)[rest], bits(case.conv_pool)[rest])


@pytest.mark.parametrize("which", ["decode_r64", "tiny_f32", "d64_g4", "d32_g2"])
def test_decode_fused_bf16_state(which):
    if which == "decode_r64":
        case, ydt = bf16_case(decode_r64()), torch.bfloat16
    elif which in ("d64_g4", "d32_g2"):
        # d = 64 with 4 value heads per key head, d = 32 with 2 (8 and 4 lanes a row)
        dims = GdnDims(2, 8, 64, 64, 4) if which == "d64_g4" else GdnDims(3, 6, 32, 32, 4)
        case = make_gdn_case(52 if which == "d64_g4" else 53, dims, [1] * 11, num_slots=17,
                             permute_slots=True, state_std=0.02, hist_std=1.0, gamma_std=0.1)
        case, ydt = bf16_case(case), torch.bfloat16
    else:
        case = make_gdn_case(51, TINY_DIMS, [1] * 9, num_slots=14, permute_slots=True,
                             act_dtype=torch.float32, state_std=0.02, hist_std=1.0, gamma_std=0.1)
        case.has_initial = torch.tensor([r % 4 != 2 for r in range(9)], dtype=torch.uint8)
        case, ydt = bf16_case(case), torch.float32
    d = case.dims
    R = case.num_reqs
    pool, state = dev(case.conv_pool), dev(case.state_pool)
    y = torch.empty((R, d.num_v_heads * d.head_dim_v), dtype=ydt, device="cuda")
    o = torch.empty((R, d.num_v_heads, d.head_dim_v), device="cuda")
    gdn.gdn_decode_fused(d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b),
                         dev(case.conv_w), dev(case.gamma), pool, state, dev(case.slot_ids), y,
                         has_initial=dev(case.has_initial), o=o, l2_eps=L2_EPS, norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    o_ref, y_ref, st_ref, pr = oracle_chain(case)
    assert rel_l2(f64(o), o_ref) <= FP32_TOL
    if ydt == torch.bfloat16:
        assert bf16_ulp_ok(y, y_ref.reshape(R, -1), ulps=1)
    else:
        assert rel_l2(f64(y), y_ref) <= FP32_TOL
    used = sorted(int(s) for s in case.slot_ids)
    check_bf16_state(state, st_ref, used, 1e-3)
    check_untouched(case, state, pool, used)


def test_spec_verify_bf16_state():
    case = bf16_case(spec_verify_r64())
    spec = case.meta["spec_slots"]
    d = case.dims
    T = case.num_tokens
    pool, state = dev(case.conv_pool), dev(case.state_pool)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((T, d.num_v_heads, d.head_dim_v), device="cuda")
    gdn.gdn_spec_verify(d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b),
                        dev(case.conv_w), dev(case.gamma), pool, state, dev(case.qsl),
                        dev(case.slot_ids), dev(spec), y, o=o, l2_eps=L2_EPS, norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    z = f64(case.z).reshape(T, d.num_v_heads, d.head_dim_v)
    y_ref, o_ref, hist_ref, st_ref = oracle.spec_verify(
        f64(case.x_qkv), z, f64(case.a), f64(case.b), f64(case.conv_w), f64(case.gamma),
        f64(case.conv_pool), f64(case.state_pool), case.qsl.numpy(), case.slot_ids.numpy(),
        spec.numpy(), case.has_initial.numpy(), d.num_k_heads, d.num_v_heads, d.head_dim_k,
        d.head_dim_v, L2_EPS, NORM_EPS)
    assert rel_l2(f64(o), o_ref) <= FP32_TOL
    assert bf16_ulp_ok(y, y_ref, ulps=1)
    written = sorted(int(s) for s in spec.flatten())
    check_bf16_state(state, st_ref, written, 1e-3)
    for s in written:
        np.testing.assert_array_equal(bits(pool)[s], bits(torch.from_numpy(hist_ref[s]).to(torch.bfloat16)))


@pytest.mark.parametrize("which", ["d128_group", "d128_group_f32y", "d128_rows", "d16_seq"])
def test_prefill_fused_bf16_state(which):
    """Packed prefill with a bf16 state: the block shapes of the chunked chain
    (whole-head blocks forming the gated output for >= 256 (request, head) units
    with a bf16 y; key-head group blocks for the same units with an fp32 y;
    32-row paired blocks for few units) and the sequential kernel (d = 16)."""
    if which in ("d128_group", "d128_group_f32y"):  # >= 256 (request, head) units
        case = make_gdn_case(61, GdnDims(4, 12, 128, 128, 4), [40, 1, 77, 33] * 6, num_slots=30,
                             permute_slots=True, state_std=0.02, hist_std=1.0, gamma_std=0.1)
    elif which == "d128_rows":  # few units: 32-row per-head blocks
        case = make_gdn_case(62, GdnDims(2, 6, 128, 128, 4), [70, 3, 129], num_slots=5,
                             permute_slots=True, state_std=0.02, hist_std=1.0, gamma_std=0.1)
    else:
        case = make_gdn_case(63, TINY_DIMS, [64, 5, 17], num_slots=6, permute_slots=True,
                             act_dtype=torch.float32, state_std=0.02, hist_std=1.0, gamma_std=0.1)
    case.has_initial = torch.tensor([r % 3 != 1 for r in range(case.num_reqs)], dtype=torch.uint8)
    case = bf16_case(case)
    d = case.dims
    T = case.num_tokens
    f32y = which.endswith("f32y")
    ydt = torch.bfloat16 if case.x_qkv.dtype == torch.bfloat16 and not f32y else torch.float32
    pool, state = dev(case.conv_pool), dev(case.state_pool)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=ydt, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_fused_workspace_bytes(d, T, case.num_reqs), dtype=torch.uint8,
                     device="cuda")
    gdn.gdn_prefill_fused(d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b),
                          dev(case.conv_w), dev(case.gamma), pool, state, dev(case.qsl),
                          dev(case.slot_ids), dev(case.has_initial), y, ws, l2_eps=L2_EPS,
                          norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    o_ref, y_ref, st_ref, pr = oracle_chain(case)
    e_y = rel_l2(f64(y), y_ref)
    print(f"{which}: y rel-L2 {e_y:.2e}")
    assert e_y <= OUT_TOL
    used = sorted(int(s) for s in case.slot_ids)
    # the chunked prefill's state error is ~5e-6 of the rms (bf16x3 contractions),
    # so near-cancelling elements may be off by a few times that in absolute terms
    check_bf16_state(state, st_ref, used, 1e-2, abs_rel=3e-5)
    for s in used:
        np.testing.assert_array_equal(bits(pool)[s], bits(torch.from_numpy(pr[s]).to(case.conv_pool.dtype)))
    check_untouched(case, state, pool, used)
