"""GPU parity of gdn_spec_verify (speculative multi-token verify) against the
fp64 oracle, through the C ABI: outputs o (fp32 copy) and y, the state and the
conv history after every token in its own slot (history bit-exact), input and
unused slots untouched."""
import numpy as np
import pytest
import torch

import oracle
from helpers import FP32_TOL, bf16_ulp_ok, bits, dev, f64, rel_l2
from hybrid_linear_attention_amd import gdn
from hybrid_linear_attention_amd.workloads import (TINY_DIMS, GdnDims, make_gdn_case,
                                                   spec_verify_r64)

pytestmark = pytest.mark.gpu

L2_EPS = 1e-6
NORM_EPS = 1e-6


def small_case(which):
    """Mixed lengths 0..max_tokens, a permuted pool with spare slots, some
    requests without an initial state, and position 0 written in place for
    every third request."""
    if which == "tiny_f32":
        dims, lens, maxn, act, ydt, seed = TINY_DIMS, [3, 1, 8, 0, 5, 2, 7, 4], 8, torch.float32, torch.float32, 41
    elif which == "d32_g2":
        dims, lens, maxn, act, ydt, seed = GdnDims(3, 6, 32, 32, 4), [5, 1, 3, 0, 5, 2], 5, torch.bfloat16, torch.bfloat16, 43
    else:
        dims, lens, maxn, act, ydt, seed = GdnDims(2, 8, 64, 64, 4), [2, 4, 1, 3, 4, 0, 4], 4, torch.bfloat16, torch.bfloat16, 42
    nreq = len(lens)
    num_slots = nreq * (maxn + 1) + 5
    case = make_gdn_case(seed, dims, lens, num_slots=num_slots, permute_slots=True,
                         act_dtype=act, state_std=0.02, hist_std=1.0, gamma_std=0.1)
    case.has_initial = torch.tensor([r % 5 != 3 for r in range(nreq)], dtype=torch.uint8)
    rng = np.random.default_rng(seed + 100)
    free = [s for s in range(num_slots) if s not in set(case.used_slots)]
    pick = rng.permutation(free)[:nreq * maxn]
    spec = torch.tensor(pick, dtype=torch.int32).reshape(nreq, maxn)
    for r in range(0, nreq, 3):
        spec[r, 0] = case.slot_ids[r]
    return case, spec, ydt


def run_gpu(case, spec, ydt):
    d = case.dims
    T = case.num_tokens
    pool = dev(case.conv_pool)
    state = dev(case.state_pool)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=ydt, device="cuda")
    o = torch.empty((T, d.num_v_heads, d.head_dim_v), device="cuda")
    gdn.gdn_spec_verify(d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b),
                        dev(case.conv_w), dev(case.gamma), pool, state, dev(case.qsl),
                        dev(case.slot_ids), dev(spec), y, has_initial=dev(case.has_initial), o=o,
                        l2_eps=L2_EPS, norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    return y, o, pool, state


def run_oracle(case, spec):
    d = case.dims
    z = f64(case.z).reshape(case.num_tokens, d.num_v_heads, d.head_dim_v)
    return oracle.spec_verify(f64(case.x_qkv), z, f64(case.a), f64(case.b), f64(case.conv_w),
                              f64(case.gamma), f64(case.conv_pool), f64(case.state_pool),
                              case.qsl.numpy(), case.slot_ids.numpy(), spec.numpy(),
                              case.has_initial.numpy(), d.num_k_heads, d.num_v_heads,
                              d.head_dim_k, d.head_dim_v, L2_EPS, NORM_EPS)


def written_slots(case, spec):
    lens = np.diff(case.qsl.numpy())
    return sorted(int(spec[r, j]) for r in range(case.num_reqs) for j in range(lens[r]))


def check(case, spec, ydt, y, o, pool, state, tol_state=FP32_TOL):
    y_ref, o_ref, hist_ref, st_ref = run_oracle(case, spec)
    e_o = rel_l2(f64(o), o_ref)
    ws = written_slots(case, spec)
    e_s = rel_l2(f64(state)[ws], st_ref[ws])
    print(f"o {e_o:.2e} states {e_s:.2e} ({len(ws)} slots)")
    assert e_o <= FP32_TOL and e_s <= tol_state
    if ydt == torch.bfloat16:
        assert bf16_ulp_ok(y, y_ref, ulps=1)
    else:
        assert rel_l2(f64(y), y_ref) <= FP32_TOL
    # history of every written slot bit-exact; every other slot untouched
    gb, ib = bits(pool), bits(case.conv_pool)
    for s in ws:
        ref = torch.from_numpy(hist_ref[s]).to(case.conv_pool.dtype)
        np.testing.assert_array_equal(gb[s], bits(ref), err_msg=f"history slot {s}")
    rest = sorted(set(range(case.num_slots)) - set(ws))
    np.testing.assert_array_equal(gb[rest], ib[rest])
    np.testing.assert_array_equal(bits(state)[rest], bits(case.state_pool)[rest])


@pytest.mark.parametrize("which", ["tiny_f32", "d64_g4", "d32_g2"])
def test_spec_verify_parity(which):
    case, spec, ydt = small_case(which)
    assert gdn.gdn_validate_spec_metadata(case.qsl, case.slot_ids, spec, case.num_tokens,
                                          case.num_slots) == 0
    y, o, pool, state = run_gpu(case, spec, ydt)
    check(case, spec, ydt, y, o, pool, state)


def test_spec_verify_full_size():
    """64 requests x 4 tokens at full shapes (the bench workload)."""
    case = spec_verify_r64()
    spec = case.meta["spec_slots"]
    y, o, pool, state = run_gpu(case, spec, torch.bfloat16)
    check(case, spec, torch.bfloat16, y, o, pool, state)


def test_spec_verify_one_token_equals_fused_decode():
    """One token per request: the same step as gdn_decode_fused, state written
    to the spec slot instead of in place."""
    case, _, _ = small_case("d64_g4")
    case = make_gdn_case(43, case.dims, [1] * 11, num_slots=30, permute_slots=True,
                         state_std=0.02, hist_std=1.0, gamma_std=0.1)
    spec = case.slot_ids.reshape(-1, 1).clone()  # in place, as the decode step
    y1, o1, pool1, state1 = run_gpu(case, spec, torch.bfloat16)
    d = case.dims
    R = case.num_reqs
    pool2, state2 = dev(case.conv_pool), dev(case.state_pool)
    y2 = torch.empty((R, d.num_v_heads * d.head_dim_v), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty((R, d.num_v_heads, d.head_dim_v), device="cuda")
    gdn.gdn_decode_fused(d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b),
                         dev(case.conv_w), dev(case.gamma), pool2, state2, dev(case.slot_ids), y2,
                         has_initial=dev(case.has_initial), o=o2, l2_eps=L2_EPS, norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(pool1), bits(pool2))
    used = sorted(int(s_) for s_ in case.slot_ids)
    unused = sorted(set(range(case.num_slots)) - set(used))
    assert rel_l2(f64(state1)[used], f64(state2)[used]) <= 1e-6
    np.testing.assert_array_equal(bits(state1)[unused], bits(state2)[unused])
    assert rel_l2(f64(o1), f64(o2)) <= 1e-6
    assert bf16_ulp_ok(y1, f64(y2), ulps=1)


def test_spec_verify_host_checks():
    case, spec, ydt = small_case("d64_g4")
    bad = spec.clone()
    bad[1, 1] = bad[2, 0]
    assert gdn.gdn_validate_spec_metadata(case.qsl, case.slot_ids, bad, case.num_tokens,
                                          case.num_slots) == 8
    d = case.dims
    y = torch.empty((case.num_tokens, d.num_v_heads * d.head_dim_v), dtype=ydt, device="cuda")
    with pytest.raises(gdn.GdnError):  # more tokens than max_tokens x requests
        gdn.gdn_spec_verify(d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b),
                            dev(case.conv_w), dev(case.gamma), dev(case.conv_pool),
                            dev(case.state_pool), dev(case.qsl), dev(case.slot_ids),
                            dev(spec[:, :1].contiguous()), y)
