"""Full-size GPU parity on sampled outputs.

The GPU runs the whole workload in the same launch configuration bench.py
times (conv1d_update -> prefill_varlen -> gated_norm over every head and
request).  The oracle then recomputes selected key-head groups (a key head and
the value heads that read it) from the same inputs: the conv is per channel and
heads never interact, so slicing the conv channels of one group is exact.
Conv history is checked bit for bit over every channel, and slots no request
uses must keep their sentinel bits.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import OUT_TOL, STATE_TOL, bits, f64, rel_l2
from hybrid_linear_attention_amd import gdn
from hybrid_linear_attention_amd.workloads import prefill_4096, prefill_varlen16

pytestmark = pytest.mark.gpu

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
    del q, k, v
    return o.cpu(), y.cpu(), pool.cpu(), state.cpu()


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
    return y.cpu(), pool.cpu(), state.cpu()


def group_channels(d, kh):
    """Conv channels of key head kh and of the value heads that read it."""
    D = d.head_dim_k
    g = d.num_v_heads // d.num_k_heads
    nq = d.num_k_heads * D
    qc = np.arange(kh * D, (kh + 1) * D)
    kc = nq + qc
    vc = 2 * nq + np.arange(kh * g * D, (kh + 1) * g * D)
    return np.concatenate([qc, kc, vc]), list(range(kh * g, (kh + 1) * g))


def oracle_group(case, kh, req_ids):
    """Oracle on key head kh's group, for the listed requests only."""
    d = case.dims
    D = d.head_dim_k
    ch, vheads = group_channels(d, kh)
    qsl = case.qsl.numpy()
    rows = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in req_ids])
    lens = [int(qsl[r + 1] - qsl[r]) for r in req_ids]
    sub_qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = case.slot_ids.numpy()[req_ids]
    hi = case.has_initial.numpy()[req_ids]
    x = f64(case.x_qkv[rows][:, ch])
    w = f64(case.conv_w[ch])
    hist = f64(case.conv_pool[:, ch])
    qq, kk, vv, _ = oracle.conv1d_update(x, w, hist, sub_qsl, slots, hi, 1, len(vheads), D, D,
                                         L2_EPS)
    a = f64(case.a[rows][:, vheads])
    b = f64(case.b[rows][:, vheads])
    st0 = f64(case.state_pool[:, vheads])
    o, st = oracle.gated_delta_rule(qq, kk, vv, a, b, st0, sub_qsl, slots, hi)
    z = f64(case.z[rows][:, vheads])
    y = oracle.gated_norm(o, z, f64(case.gamma), NORM_EPS)
    return rows, vheads, o, y, st, slots


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
    # requests with L >= 3 never read their old history for the new one, but the
    # oracle's window still starts with it; rows before them are irrelevant.
    _, new = oracle.conv1d_silu(f64(case.x_qkv[rows]), f64(case.conv_w), f64(case.conv_pool),
                                sub_qsl, case.slot_ids.numpy(), case.has_initial.numpy())
    return new


def check_common(case, o, y, pool, state, groups, req_ids):
    for kh in groups:
        rows, vheads, o_ref, y_ref, st_ref, slots = oracle_group(case, kh, req_ids)
        e_o = rel_l2(f64(o[rows][:, vheads]), o_ref) if o is not None else 0.0
        D = case.dims.head_dim_v
        yv = f64(y[rows].reshape(len(rows), case.dims.num_v_heads, D)[:, vheads])
        e_y = rel_l2(yv, y_ref.reshape(len(rows), len(vheads), D))
        e_s = rel_l2(f64(state[slots][:, vheads]), st_ref[slots])
        print(f"key head {kh}: o {e_o:.2e}  y {e_y:.2e}  state {e_s:.2e}")
        assert e_o <= OUT_TOL and e_y <= OUT_TOL and e_s <= STATE_TOL
    new_hist = expected_history(case)
    used = set(int(s) for s in case.slot_ids)
    gb, ib = bits(pool), bits(case.conv_pool)
    for s in range(case.num_slots):
        if s in used:
            ref = torch.from_numpy(new_hist[s]).to(case.conv_pool.dtype)
            np.testing.assert_array_equal(gb[s], bits(ref), err_msg=f"history slot {s}")
        else:
            np.testing.assert_array_equal(gb[s], ib[s], err_msg=f"unused history slot {s}")
    unused = sorted(set(range(case.num_slots)) - used)
    if unused:
        np.testing.assert_array_equal(bits(state)[unused], bits(case.state_pool)[unused])


def test_prefill_4096_sampled():
    case = prefill_4096()
    o, y, pool, state = run_chain_gpu(case)
    check_common(case, o, y, pool, state, groups=[0, 7, 15], req_ids=[0])


def test_prefill_varlen16_sampled():
    case = prefill_varlen16()
    o, y, pool, state = run_chain_gpu(case)
    lens = np.diff(case.qsl.numpy())
    longest = int(np.argmax(lens))
    shortest = int(np.argmin(lens))
    reqs = sorted({0, longest, shortest, case.num_reqs - 1})
    check_common(case, o, y, pool, state, groups=[3, 12], req_ids=reqs)


def test_prefill_4096_fused_sampled():
    case = prefill_4096()
    y, pool, state = run_fused_gpu(case)
    check_common(case, None, y, pool, state, groups=[2, 9], req_ids=[0])


def test_prefill_varlen16_fused_sampled():
    case = prefill_varlen16()
    y, pool, state = run_fused_gpu(case)
    lens = np.diff(case.qsl.numpy())
    reqs = sorted({0, int(np.argmax(lens)), int(np.argmin(lens)), case.num_reqs - 1})
    check_common(case, None, y, pool, state, groups=[5, 14], req_ids=reqs)
