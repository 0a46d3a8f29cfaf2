"""gdn_prefill_fused_noalloc against gdn_prefill_fused, through the C ABI.

The no-allocation entry point runs the same kernels as gdn_prefill_fused on the
library's static per-GPU scratch instead of a caller workspace, so on the same
inputs every output, state and history bit must equal the workspace call's.
Two calls in a row, the second on a smaller batch (the scratch then holds the
first call's leftovers, which nothing may read), and a batch beyond the
scratch's size, which must be refused before anything runs.
"""
import numpy as np
import pytest
import torch

from helpers import OUT_TOL, bits, dev, f64, rel_l2
from hybrid_linear_attention_amd import gdn
from hybrid_linear_attention_amd.workloads import FULL_DIMS, make_gdn_case

pytestmark = pytest.mark.gpu

L2_EPS = 1e-6
NORM_EPS = 1e-6


def run(case, noalloc):
    d = case.dims
    T = case.num_tokens
    pool, state = dev(case.conv_pool), dev(case.state_pool)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=torch.bfloat16, device="cuda")
    args = (d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b), dev(case.conv_w),
            dev(case.gamma), pool, state, dev(case.qsl), dev(case.slot_ids), dev(case.has_initial), y)
    if noalloc:
        gdn.gdn_prefill_fused_noalloc(*args, l2_eps=L2_EPS, norm_eps=NORM_EPS)
    else:
        ws = torch.empty(gdn.gdn_prefill_fused_workspace_bytes(d, T, case.num_reqs),
                         dtype=torch.uint8, device="cuda")
        gdn.gdn_prefill_fused(*args, ws, l2_eps=L2_EPS, norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    return [y.cpu(), pool.cpu(), state.cpu()]


def test_noalloc_matches_workspace_call_twice():
    # first a large batch (32-row chain blocks: 3 requests x 48 heads < 256),
    # then a smaller one in more requests (whole-head chain blocks that form the
    # gated output)
    cases = [make_gdn_case(701, FULL_DIMS, [1200, 77, 700], num_slots=6, permute_slots=True,
                           state_std=0.02, hist_std=1.0, gamma_std=0.1),
             make_gdn_case(702, FULL_DIMS, [40, 5, 0, 33, 1, 64], num_slots=9, permute_slots=True,
                           state_std=0.02, hist_std=1.0, gamma_std=0.1)]
    for i, case in enumerate(cases):
        need = gdn.gdn_prefill_fused_workspace_bytes(case.dims, case.num_tokens, case.num_reqs)
        assert need <= gdn.GDN_NOALLOC_SCRATCH_BYTES
        print(f"call {i}: {case.num_tokens} tokens, {case.num_reqs} requests, "
              f"scratch {need / 2**20:.1f} MiB", flush=True)
        ref = run(case, noalloc=False)
        got = run(case, noalloc=True)
        for name, g, r in zip(("y", "history", "state"), got, ref):
            np.testing.assert_array_equal(bits(g), bits(r), err_msg=f"call {i}: {name}")
        # and the step did run: y is not the untouched buffer, and matches itself
        assert rel_l2(f64(got[0]), f64(ref[0])) <= OUT_TOL and float(f64(got[0]).std()) > 0


def test_noalloc_refuses_a_batch_beyond_its_scratch():
    case = make_gdn_case(703, FULL_DIMS, [8], num_slots=1)
    T = 4096  # ~344 MiB of scratch in one request
    assert gdn.gdn_prefill_fused_workspace_bytes(FULL_DIMS, T, 1) > gdn.GDN_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, FULL_DIMS.conv_channels), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros((T, 48, 128), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((T, 48), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, 48 * 128), dtype=torch.bfloat16, device="cuda")
    pool, state = dev(case.conv_pool), dev(case.state_pool)
    qsl = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(gdn.GdnError) as err:
        gdn.gdn_prefill_fused_noalloc(FULL_DIMS, x, z, a, a.clone(), dev(case.conv_w), dev(case.gamma),
                                      pool, state, qsl, dev(case.slot_ids), None, y)
    assert err.value.status == 9  # GDN_ERR_SCRATCH
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(state.cpu()), bits(case.state_pool))
