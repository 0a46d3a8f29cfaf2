"""GPU parity of the full GDN layer block on the mixed batch at hidden 5120
(8 prefill requests of 2048 tokens, then 256 one-token decode requests).

The GPU runs the whole layer once, in the launch sequence bench.py times.  The
oracle then checks:
  * each stage on every row, fed the GPU's own input to that stage (RMSNorm,
    in-projection, out-projection + residual: one bf16 rounding each);
  * the GDN core (conv, prefill and decode recurrence, gated norm) on every
    key-head group and every request, fed the GPU's bf16 projection output,
    against the output and state tolerances and the row bounds;
  * the conv history of every slot, bit for bit;
  * end to end: the full fp64 layer on a sub-batch (one prefill request and a
    few decode requests; requests are independent), on the mixer output Y - X.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (OUT_TOL, STATE_TOL, bf16_ulp_ok, bits, check_o_rows, check_y_rows, f64,
                     rel_l2)
from hybrid_linear_attention_amd.layer import GdnLayer, stack_weights
from hybrid_linear_attention_amd.workloads import layer_mixed

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

EPS = 1e-6
# End-to-end bound on the mixer output Y - X against the unrounded fp64 chain: the
# GPU rounds U, the projection, y and Y to bf16 (2^-9 relative each) and the
# conv / L2 norm / recurrence carry the projection's rounding through; 1e-2 is
# about three times the sum of those contributions.
E2E_TOL = 1e-2


@pytest.fixture(scope="module", params=[True, False], ids=["fused", "separate"])
def layer_run(request):
    """The layer with the core through gdn_prefill_fused / gdn_decode_fused, and
    through the separate conv / prefill / decode / gated-norm entry points."""
    fused = request.param
    case = layer_mixed()
    core = case.core
    d = core.dims
    T = int(core.qsl[-1])
    w = stack_weights(d, case.W_qkvz, case.W_ba, case.W_o, core.conv_w, case.gamma_in,
                      core.gamma)
    T_pf = case.num_prefill * case.prefill_len
    layer = GdnLayer(d, w, T, case.num_prefill, T_pf, case.num_decode, EPS, EPS, fused=fused)
    X = case.X.cuda()
    pool = core.conv_pool.cuda()
    state = core.state_pool.cuda()
    print(f"layer block: T={T} prefill={case.num_prefill}x{case.prefill_len} "
          f"decode={case.num_decode}", flush=True)
    layer.forward(X, pool, state, core.qsl.cuda(), core.slot_ids.cuda(),
                  core.has_initial.cuda())
    torch.cuda.synchronize()
    out = dict(U=layer.U.cpu(), P=layer.P.cpu(), o=None if fused else layer.o.cpu(),
               y=layer.y.cpu(), Y=layer.Y.cpu(), pool=pool.cpu(), state=state.cpu(),
               W_in=w.W_in.cpu(), cq=layer.cq, cz=layer.cz, T=T, T_pf=T_pf)
    del layer, X, pool, state, w
    torch.cuda.empty_cache()
    return case, out


ROW_BLOCK = 2048


def test_layer_rmsnorm_and_projections(layer_run):
    """Every row of U, of the in-projection output and of Y, in blocks of rows."""
    case, g = layer_run
    T = g["T"]
    W_in = f64(g["W_in"]).T
    W_in_ref = np.concatenate([f64(case.W_qkvz), f64(case.W_ba)], axis=1)
    np.testing.assert_array_equal(W_in, W_in_ref)
    W_o = f64(case.W_o)
    gamma_in = f64(case.gamma_in)
    for r0 in range(0, T, ROW_BLOCK):
        rows = slice(r0, min(T, r0 + ROW_BLOCK))
        X = f64(case.X[rows])
        U_ref = oracle.rmsnorm(X, gamma_in, EPS)
        assert bf16_ulp_ok(g["U"][rows], U_ref), f"U rows {rows}"
        # in-projection fed the GPU's U: columns q|k|v|z|b|a
        P_ref = oracle.linear(f64(g["U"][rows]), W_in)
        assert bf16_ulp_ok(g["P"][rows], P_ref), f"P rows {rows}"
        # out-projection + residual fed the GPU's y
        Y_ref = oracle.residual_add(X, oracle.linear(f64(g["y"][rows]), W_o))
        assert bf16_ulp_ok(g["Y"][rows], Y_ref), f"Y rows {rows}"
        print(f"rows {r0}..{rows.stop - 1}: U, P, Y within one rounding", flush=True)


def _group(d, kh):
    D = d.head_dim_k
    gsz = d.num_v_heads // d.num_k_heads
    nq = d.num_k_heads * D
    qc = np.arange(kh * D, (kh + 1) * D)
    vc = 2 * nq + np.arange(kh * gsz * D, (kh + 1) * gsz * D)
    return np.concatenate([qc, nq + qc, vc]), list(range(kh * gsz, (kh + 1) * gsz))


@pytest.mark.parametrize("kh", list(range(16)))
def test_layer_core_groups(layer_run, kh):
    """Key head kh's group over every request of the mixed batch."""
    case, g = layer_run
    core = case.core
    d = core.dims
    D = d.head_dim_k
    Hv = d.num_v_heads
    ch, vheads = _group(d, kh)
    qsl = core.qsl.numpy()
    slots = core.slot_ids.numpy()
    hi = core.has_initial.numpy()
    T = g["T"]
    cq, cz = g["cq"], g["cz"]
    x = f64(g["P"][:, ch])
    zc = np.concatenate([cq + h * D + np.arange(D) for h in vheads])
    z = f64(g["P"][:, zc]).reshape(T, len(vheads), D)
    b = f64(g["P"][:, [cq + cz + h for h in vheads]])
    a = f64(g["P"][:, [cq + cz + Hv + h for h in vheads]])
    qq, kk, vv, _ = oracle.conv1d_update(x, f64(core.conv_w[ch]), f64(core.conv_pool[:, ch]),
                                         qsl, slots, hi, 1, len(vheads), D, D, EPS)
    o_ref, st_ref = oracle.gated_delta_rule(qq, kk, vv, a, b, f64(core.state_pool[:, vheads]),
                                            qsl, slots, hi)
    y_ref = oracle.gated_norm(o_ref, z, f64(core.gamma), EPS).reshape(T, len(vheads), D)
    y = f64(g["y"].reshape(T, Hv, D)[:, vheads])
    st = f64(g["state"][:, vheads])
    npf = g["T_pf"]
    pf_slots = slots[:case.num_prefill]
    dec_slots = slots[case.num_prefill:]
    e = dict(y_prefill=rel_l2(y[:npf], y_ref[:npf]), y_decode=rel_l2(y[npf:], y_ref[npf:]),
             state_prefill=rel_l2(st[pf_slots], st_ref[pf_slots]),
             state_decode=rel_l2(st[dec_slots], st_ref[dec_slots]))
    e["y_row"] = check_y_rows(y, y_ref, o_ref, z, f64(core.gamma), D)
    if g["o"] is not None:
        o = f64(g["o"][:, vheads])
        e.update(o_prefill=rel_l2(o[:npf], o_ref[:npf]), o_decode=rel_l2(o[npf:], o_ref[npf:]))
        e["o_row"] = check_o_rows(o, o_ref, D)
    print(f"key head {kh}: " + "  ".join(f"{k} {v:.2e}" for k, v in e.items()))
    assert all(v <= OUT_TOL for k, v in e.items() if k[0] in "oy" and not k.endswith("_row"))
    assert e["state_prefill"] <= STATE_TOL and e["state_decode"] <= STATE_TOL


def test_layer_history_bits(layer_run):
    """New history of every slot from each request's last (up to) three rows of
    the GPU's projection output."""
    case, g = layer_run
    core = case.core
    qsl = core.qsl.numpy()
    rows, lens = [], []
    for r in range(core.num_reqs):
        m = min(int(qsl[r + 1] - qsl[r]), 3)
        rows.append(np.arange(qsl[r + 1] - m, qsl[r + 1]))
        lens.append(m)
    rows = np.concatenate(rows)
    sub_qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = f64(g["P"][rows][:, :g["cq"]])
    _, new = oracle.conv1d_silu(x, f64(core.conv_w), f64(core.conv_pool), sub_qsl,
                                core.slot_ids.numpy(), core.has_initial.numpy())
    ref = torch.from_numpy(new).to(core.conv_pool.dtype)
    np.testing.assert_array_equal(bits(g["pool"]), bits(ref))


def test_layer_end_to_end(layer_run):
    """Full fp64 layer on prefill request 0 plus decode requests 0..7 of the batch."""
    case, g = layer_run
    core = case.core
    d = core.dims
    qsl = core.qsl.numpy()
    reqs = [0] + list(range(case.num_prefill, case.num_prefill + 8))
    rows = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in reqs])
    lens = [int(qsl[r + 1] - qsl[r]) for r in reqs]
    sub_qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = core.slot_ids.numpy()[reqs]
    Xs = f64(case.X[rows])
    # the sub-batch's slots, renumbered 0..len(reqs)-1
    Y_ref, _, st_ref, _ = oracle.gdn_layer(
        Xs, f64(case.gamma_in), f64(case.W_qkvz), f64(case.W_ba), f64(core.conv_w),
        f64(core.gamma), f64(case.W_o), f64(core.conv_pool[slots]), f64(core.state_pool[slots]),
        sub_qsl, np.arange(len(reqs), dtype=np.int32), core.has_initial.numpy()[reqs],
        d.num_k_heads, d.num_v_heads, d.head_dim_k, d.head_dim_v, EPS, EPS)
    Y = f64(g["Y"][rows])
    e_mix = rel_l2(Y - Xs, Y_ref - Xs)
    e_st = rel_l2(f64(g["state"][slots]), st_ref)
    print(f"end to end: mixer output rel-L2 {e_mix:.2e}, states {e_st:.2e}")
    assert e_mix <= E2E_TOL
    assert e_st <= E2E_TOL
