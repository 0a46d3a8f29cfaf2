"""Full-size GPU parity on the whole output.

The GPU runs each full-size prefill workload twice, in the launch
configurations bench.py times: through the separate entry points
(conv1d_update -> prefill_varlen -> gated_norm, which leaves o visible) and
through gdn_prefill_fused.  The oracle then recomputes every key-head group (a
key head and the value heads that read it) over every request from the same
inputs: the conv is per channel and heads never interact, so slicing the conv
channels of one group is exact.  Every group must meet the output and state
tolerances, every (token, head) row its row bound, the conv history of every
slot must match bit for bit, and slots no request uses keep their sentinel bits.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (OUT_TOL, STATE_TOL, bits, check_o_rows, check_y_rows, f64, rel_l2)
from hybrid_linear_attention_amd import gdn
from hybrid_linear_attention_amd.workloads import prefill_4096, prefill_varlen16

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

L2_EPS = 1e-6
NORM_EPS = 1e-6


def run_chain_gpu(case):
    d = case.dims
    T = case.num_tokens
    D = d.head_dim_k
    q = torch.empty((T, d.num_k_heads, D), device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((T, d.num_v_heads, D), device="cuda")
    o = torch.empty((T, d.num_v_heads, D), device="cuda")
    y = torch.empty((T, d.num_v_heads * D), dtype=torch.bfloat16, device="cuda")
    pool = case.conv_pool.cuda()
    state = case.state_pool.cuda()
    qsl, slots, hi = case.qsl.cuda(), case.slot_ids.cuda(), case.has_initial.cuda()
    gdn.gdn_conv1d_update(d, case.x_qkv.cuda(), case.conv_w.cuda(), pool, qsl, slots, hi, q, k, v,
                          l2_eps=L2_EPS)
    nbytes = gdn.gdn_prefill_workspace_bytes(d, T, case.num_reqs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
    gdn.gdn_prefill_varlen(d, q, k, v, case.a.cuda(), case.b.cuda(), state, qsl, slots, hi, o, ws)
    gdn.gdn_gated_norm(d, o, case.z.cuda(), case.gamma.cuda(), y, eps=NORM_EPS)
    torch.cuda.synchronize()
    del q, k, v, ws
    return dict(o=o.cpu(), y=y.cpu(), pool=pool.cpu(), state=state.cpu())


def run_fused_gpu(case):
    """The same step through the one-call fused entry point."""
    d = case.dims
    T = case.num_tokens
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=torch.bfloat16, device="cuda")
    pool = case.conv_pool.cuda()
    state = case.state_pool.cuda()
    nbytes = gdn.gdn_prefill_fused_workspace_bytes(d, T, case.num_reqs)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    gdn.gdn_prefill_fused(d, case.x_qkv.cuda(), case.z.cuda(), case.a.cuda(), case.b.cuda(),
                          case.conv_w.cuda(), case.gamma.cuda(), pool, state, case.qsl.cuda(),
                          case.slot_ids.cuda(),
                          case.has_initial.cuda(), y, ws, l2_eps=L2_EPS, norm_eps=NORM_EPS)
    torch.cuda.synchronize()
    del ws
    return dict(o=None, y=y.cpu(), pool=pool.cpu(), state=state.cpu())


def group_channels(d, kh):
    """Conv channels of key head kh and of the value heads that read it."""
    D = d.head_dim_k
    g = d.num_v_heads // d.num_k_heads
    nq = d.num_k_heads * D
    qc = np.arange(kh * D, (kh + 1) * D)
    kc = nq + qc
    vc = 2 * nq + np.arange(kh * g * D, (kh + 1) * g * D)
    return np.concatenate([qc, kc, vc]), list(range(kh * g, (kh + 1) * g))


def oracle_group(case, kh):
    """Oracle on key head kh's group over every request."""
    d = case.dims
    D = d.head_dim_k
    ch, vheads = group_channels(d, kh)
    qsl = case.qsl.numpy()
    slots = case.slot_ids.numpy()
    hi = case.has_initial.numpy()
    qq, kk, vv, _ = oracle.conv1d_update(f64(case.x_qkv[:, ch]), f64(case.conv_w[ch]),
                                         f64(case.conv_pool[:, ch]), qsl, slots, hi, 1,
                                         len(vheads), D, D, L2_EPS)
    a = f64(case.a[:, vheads])
    b = f64(case.b[:, vheads])
    o, st = oracle.gated_delta_rule(qq, kk, vv, a, b, f64(case.state_pool[:, vheads]), qsl, slots,
                                    hi)
    z = f64(case.z[:, vheads])
    y = oracle.gated_norm(o, z, f64(case.gamma), NORM_EPS)
    return vheads, o, y, z, st


def expected_history(case):
    """New conv history over every channel: the oracle conv run on each request's
    last (up to) three rows, which determine the history exactly."""
    qsl = case.qsl.numpy()
    rows, lens = [], []
    for r in range(case.num_reqs):
        L = int(qsl[r + 1] - qsl[r])
        m = min(L, 3)
        rows.append(np.arange(qsl[r + 1] - m, qsl[r + 1]))
        lens.append(m)
    rows = np.concatenate(rows)
    sub_qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    _, new = oracle.conv1d_silu(f64(case.x_qkv[rows]), f64(case.conv_w), f64(case.conv_pool),
                                sub_qsl, case.slot_ids.numpy(), case.has_initial.numpy())
    return new


def check_history_and_slots(case, run, new_hist):
    used = set(int(s) for s in case.slot_ids)
    gb, ib = bits(run["pool"]), bits(case.conv_pool)
    for s in range(case.num_slots):
        if s in used:
            ref = torch.from_numpy(new_hist[s]).to(case.conv_pool.dtype)
            np.testing.assert_array_equal(gb[s], bits(ref), err_msg=f"history slot {s}")
        else:
            np.testing.assert_array_equal(gb[s], ib[s], err_msg=f"unused history slot {s}")
    unused = sorted(set(range(case.num_slots)) - used)
    if unused:
        np.testing.assert_array_equal(bits(run["state"])[unused], bits(case.state_pool)[unused])


def check_whole_output(case):
    d = case.dims
    D = d.head_dim_v
    T = case.num_tokens
    runs = {"separate": run_chain_gpu(case), "fused": run_fused_gpu(case)}
    print(f"{T} tokens, {case.num_reqs} requests: GPU done", flush=True)
    slots = case.slot_ids.numpy()
    worst = {name: dict(o=0.0, y=0.0, state=0.0, o_row=0.0, y_row=0.0) for name in runs}
    for kh in range(d.num_k_heads):
        vheads, o_ref, y_ref, z, st_ref = oracle_group(case, kh)
        y_ref = y_ref.reshape(T, len(vheads), D)
        for name, run in runs.items():
            yv = f64(run["y"].reshape(T, d.num_v_heads, D)[:, vheads])
            e = dict(y=rel_l2(yv, y_ref),
                     state=rel_l2(f64(run["state"][slots][:, vheads]), st_ref[slots]))
            e["y_row"] = check_y_rows(yv, y_ref, o_ref, z, f64(case.gamma), D)
            if run["o"] is not None:
                ov = f64(run["o"][:, vheads])
                e["o"] = rel_l2(ov, o_ref)
                e["o_row"] = check_o_rows(ov, o_ref, D)
            for key, val in e.items():
                worst[name][key] = max(worst[name][key], val)
            assert e.get("o", 0.0) <= OUT_TOL and e["y"] <= OUT_TOL and e["state"] <= STATE_TOL, \
                f"{name} key head {kh}: {e}"
        print(f"key head {kh:2d} done", flush=True)
    for name in runs:
        print(f"{name}: worst over groups " + "  ".join(f"{k} {v:.2e}" for k, v in worst[name].items()))
    new_hist = expected_history(case)
    for run in runs.values():
        check_history_and_slots(case, run, new_hist)


def test_prefill_4096_whole_output():
    check_whole_output(prefill_4096())


def test_prefill_varlen16_whole_output():
    check_whole_output(prefill_varlen16())
