"""GPU parity of gqa_decode_paged (GQA decode over a paged KV cache) against the
fp64 oracle (oracle.gqa_decode_paged), through the C ABI.

Bars: o (fp32, before the gate) within FP32_TOL rel-L2 (the scores keep fp32
accuracy: q enters the matrix cores as three bf16 terms against the exact bf16
K); y within one bf16 ulp where stored as bf16, FP32_TOL where fp32; the K/V
cache bit for bit (the rotated k is rounded once to bf16 on both sides from
fp64, v is copied; an e4m3 cache gets the codes nearest to k / k_scale and
v / v_scale, the same on both sides since both round the same fp64 value), every
position other than the new tokens' untouched."""
import numpy as np
import pytest
import torch

import oracle
from helpers import FP32_TOL, bf16_ulp_ok, bits, dev, f64, rel_l2
from hybrid_linear_attention_amd import gqa
from hybrid_linear_attention_amd.workloads import GqaDims, gqa_decode_r64, gqa_decode_r64_fp8, make_gqa_case

pytestmark = pytest.mark.gpu


def is_fp8(case):
    return case.k_cache.dtype == torch.uint8


def cache_values(case):
    """The values the caches hold (fp64), decoded from e4m3 codes for an fp8 cache."""
    if is_fp8(case):
        return (case.k_scale * oracle.e4m3_decode(case.k_cache.numpy()),
                case.v_scale * oracle.e4m3_decode(case.v_cache.numpy()))
    return f64(case.k_cache), f64(case.v_cache)


def run_gpu(case, y_dtype=torch.bfloat16):
    d = case.dims
    R = case.num_reqs
    kc, vc = dev(case.k_cache), dev(case.v_cache)
    y = torch.empty((R, d.num_q_heads * d.head_dim), dtype=y_dtype, device="cuda")
    o = torch.empty((R, d.num_q_heads, d.head_dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(d, R, case.max_context_len), dtype=torch.uint8,
                     device="cuda")
    gqa.gqa_decode_paged(d, dev(case.q), dev(case.gate), dev(case.k), dev(case.v), kc, vc,
                         dev(case.block_tables), dev(case.context_lens), case.page_size,
                         case.max_context_len, y, ws, rope_theta=case.rope_theta, o=o,
                         k_scale=case.k_scale, v_scale=case.v_scale)
    torch.cuda.synchronize()
    return y, o, kc, vc


def run_oracle(case, reqs=None):
    d = case.dims
    sel = slice(None) if reqs is None else reqs
    kc, vc = cache_values(case)
    rounding = {}
    if is_fp8(case):
        rounding = dict(cache_round=oracle.fp8_cache_round(case.k_scale),
                        v_round=oracle.fp8_cache_round(case.v_scale))
    return oracle.gqa_decode_paged(
        f64(case.q)[sel], f64(case.k)[sel], f64(case.v)[sel], f64(case.gate)[sel], kc, vc,
        case.block_tables.numpy()[sel], case.context_lens.numpy()[sel], case.page_size, d.rotary_dim,
        case.rope_theta, **rounding)


def check_fp8_caches(case, kc, vc, kc_ref, vc_ref, reqs):
    """e4m3 caches: the new tokens' codes equal the oracle's (its stored values
    encoded back), every other code is untouched."""
    got_k, got_v = kc.cpu().numpy(), vc.cpu().numpy()
    exp_k, exp_v = case.k_cache.numpy().copy(), case.v_cache.numpy().copy()
    P = case.page_size
    for r in reqs:
        L = int(case.context_lens[r])
        p, off = int(case.block_tables[r, (L - 1) // P]), (L - 1) % P
        exp_k[p, :, off] = oracle.e4m3_encode(kc_ref[p, :, off] / case.k_scale)
        exp_v[p, :, off] = oracle.e4m3_encode(vc_ref[p, :, off] / case.v_scale)
    np.testing.assert_array_equal(got_k, exp_k)
    np.testing.assert_array_equal(got_v, exp_v)


def check(case, y, o, kc, vc, y_dtype=torch.bfloat16):
    d = case.dims
    R = case.num_reqs
    y_ref, o_ref, kc_ref, vc_ref = run_oracle(case)
    e_o = rel_l2(f64(o), o_ref)
    print(f"o rel-L2 {e_o:.2e}")
    assert e_o <= FP32_TOL
    if y_dtype == torch.bfloat16:
        assert bf16_ulp_ok(y, y_ref.reshape(R, -1), ulps=1)
    else:
        assert rel_l2(f64(y), y_ref.reshape(R, -1)) <= FP32_TOL
    if is_fp8(case):
        check_fp8_caches(case, kc, vc, kc_ref, vc_ref, range(R))
    else:
        np.testing.assert_array_equal(bits(kc), bits(torch.from_numpy(kc_ref).to(torch.bfloat16)))
        np.testing.assert_array_equal(bits(vc), bits(torch.from_numpy(vc_ref).to(torch.bfloat16)))


FP8 = torch.float8_e4m3fn


@pytest.mark.parametrize("which", ["pages16", "pages1", "pages100", "g8_f32", "g1_norope",
                                   "fp8_pages16", "fp8_scaled", "fp8_g8_f32"])
def test_gqa_decode_parity(which):
    y_dtype = torch.bfloat16
    if which == "pages16":     # lengths around the 16-position tiles and 512-position runs (the
        # new token alone in its run at 513 and 1025: that block appends, then reads only it)
        case = make_gqa_case(81, [1, 2, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1025, 700, 64], 16)
    elif which == "pages1":    # every position on a page of its own
        case = make_gqa_case(82, [1, 3, 40, 300], 1)
    elif which == "pages100":  # a page size that is no power of two, a tile straddling pages
        case = make_gqa_case(83, [530, 1, 1200, 99, 101], 100)
    elif which == "g8_f32":    # 8 query heads per kv head, fp32 activations and y, all dims rotated
        case = make_gqa_case(84, [33, 513, 7], 16, dims=GqaDims(16, 2, 256, 256),
                             act_dtype=torch.float32)
        y_dtype = torch.float32
    elif which == "g1_norope":  # one query head per kv head, no rotation
        case = make_gqa_case(85, [20, 290], 32, dims=GqaDims(8, 8, 256, 0))
    elif which == "fp8_pages16":  # e4m3 cache at scale 1
        case = make_gqa_case(87, [1, 2, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1025, 700, 64], 16,
                             cache_dtype=FP8)
    elif which == "fp8_scaled":   # e4m3 cache with per-cache scales, a page size that is no power of two
        case = make_gqa_case(88, [530, 1, 1200, 99], 100, cache_dtype=FP8, k_scale=0.0625, v_scale=0.75)
    else:                         # e4m3 cache, 8 query heads per kv head, fp32 activations and y
        case = make_gqa_case(89, [33, 513, 7], 16, dims=GqaDims(16, 2, 256, 256), act_dtype=torch.float32,
                             cache_dtype=FP8, k_scale=2.0, v_scale=0.5)
        y_dtype = torch.float32
    assert gqa.gqa_validate_decode_metadata(case.block_tables, case.context_lens,
                                            case.k_cache.shape[0], case.page_size,
                                            case.max_context_len) == 0
    y, o, kc, vc = run_gpu(case, y_dtype)
    check(case, y, o, kc, vc, y_dtype)


@pytest.mark.parametrize("hq,hkv,rd,fp8", [(4, 2, 64, False), (6, 2, 32, False), (8, 2, 128, True),
                                          (5, 1, 64, False), (7, 1, 2, True)])
def test_gqa_decode_head_ratios(hq, hkv, rd, fp8):
    """The query heads per key/value head the kernel is built for beside 1, 6
    and 8 (2, 3, 4, 5, 7), each with the new token alone in its run (513) and
    at a page's first position (17), on a bf16 or an e4m3 cache."""
    kw = dict(cache_dtype=FP8, k_scale=0.5, v_scale=2.0) if fp8 else {}
    case = make_gqa_case(100 + hq * 8 + hkv, [513, 17, 1, 300], 16, dims=GqaDims(hq, hkv, 256, rd), **kw)
    y, o, kc, vc = run_gpu(case)
    check(case, y, o, kc, vc)


def test_gqa_skipped_request_and_slack_context_bound():
    """A request whose length is 0 is skipped (zero rows, cache untouched) and
    max_context_len may exceed every length (extra runs of positions exit)."""
    case = make_gqa_case(86, [40, 5, 300], 16, max_context_len=1000)
    lens = case.context_lens.clone()
    case.context_lens[1] = 0
    y, o, kc, vc = run_gpu(case)
    keep = [0, 2]
    y_ref, o_ref, kc_ref, vc_ref = run_oracle(case, reqs=keep)
    assert rel_l2(f64(o)[keep], o_ref) <= FP32_TOL
    assert bf16_ulp_ok(y[keep], y_ref.reshape(2, -1), ulps=1)
    assert not torch.any(y[1]).item() and not torch.any(o[1]).item()
    np.testing.assert_array_equal(bits(kc), bits(torch.from_numpy(kc_ref).to(torch.bfloat16)))
    np.testing.assert_array_equal(bits(vc), bits(torch.from_numpy(vc_ref).to(torch.bfloat16)))
    assert int(lens[1]) == 5


@pytest.mark.parametrize("which", ["long_single", "pages528_fp8"])
def test_gqa_decode_long_contexts(which):
    """One request with a 20,000-position context (79 runs merged by the
    combine) beside a 1-position one; pages of 528 positions (longer than a
    run, no power of two) on an e4m3 cache."""
    if which == "long_single":
        case = make_gqa_case(90, [20000, 1], 64)
    else:
        case = make_gqa_case(91, [3000, 528, 529, 1], 528, cache_dtype=FP8, k_scale=0.5, v_scale=1.5)
    y, o, kc, vc = run_gpu(case)
    check(case, y, o, kc, vc)


def test_gqa_decode_full_size():
    """The benchmarked workload (64 requests, 1024-3072 positions, pages of 16),
    launched as the benchmark launches it, against the oracle on every request."""
    case = gqa_decode_r64()
    y, o, kc, vc = run_gpu(case)
    check(case, y, o, kc, vc)


def test_gqa_decode_full_size_fp8():
    """The benchmarked fp8 workload (the same 64 requests, e4m3 cache)."""
    case = gqa_decode_r64_fp8()
    y, o, kc, vc = run_gpu(case)
    check(case, y, o, kc, vc)
