"""GPU parity of gdn_prefill_fused's prefix-cache snapshots against the fp64
oracle (oracle.prefill_snapshots), through the C ABI: outputs, final states,
the state after every snap_interval tokens in its snapshot slot, snapshot
histories bit-exact, every other slot untouched.  Every chain block shape takes
snapshots: whole-head blocks forming the gated output (>= 256 (request, head)
units, bf16 y), key-head group blocks (the same units with an fp32 y), 32-row
paired blocks (few units) and the sequential kernel (d = 16)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import OUT_TOL, STATE_TOL, bits, check_bf16_state, dev, f64, rel_l2
from hybrid_linear_attention_amd import gdn
from hybrid_linear_attention_amd.workloads import TINY_DIMS, GdnDims, make_gdn_case

pytestmark = pytest.mark.gpu

L2_EPS = 1e-6
NORM_EPS = 1e-6


def snap_case(which):
    if which in ("d128_group", "d128_group_f32y"):  # >= 256 (request, head) units
        dims, lens, interval, max_snaps, seed = GdnDims(4, 12, 128, 128, 4), [200, 64, 31, 96, 130] * 5, 64, 3, 71
    elif which == "d128_rows":    # few units: 32-row per-head blocks
        dims, lens, interval, max_snaps, seed = GdnDims(2, 6, 128, 128, 4), [100, 64, 32, 5], 32, 4, 72
    else:                         # d = 16: the sequential kernel
        dims, lens, interval, max_snaps, seed = TINY_DIMS, [64, 40, 7], 32, 2, 73
    act = torch.float32 if dims.head_dim_k == 16 else torch.bfloat16
    nreq = len(lens)
    num_slots = nreq * (max_snaps + 1) + 3
    case = make_gdn_case(seed, dims, lens, num_slots=num_slots, permute_slots=True, act_dtype=act,
                         state_std=0.02, hist_std=1.0, gamma_std=0.1)
    case.has_initial = torch.tensor([r % 4 != 1 for r in range(nreq)], dtype=torch.uint8)
    rng = np.random.default_rng(seed + 7)
    free = [s for s in range(num_slots) if s not in set(case.used_slots)]
    snaps = torch.tensor(rng.permutation(free)[:nreq * max_snaps], dtype=torch.int32).reshape(nreq, max_snaps)
    return case, snaps, interval


def run(case, snaps, interval, f32y=False):
    """gdn_prefill_fused with snapshots; a bf16 y for bf16 inputs unless f32y
    (an fp32 y sends >= 256 units to the key-head group blocks and the separate
    gated-norm pass instead of whole-head blocks)."""
    d = case.dims
    T = case.num_tokens
    ydt = torch.bfloat16 if case.x_qkv.dtype == torch.bfloat16 and not f32y else torch.float32
    pool, state = dev(case.conv_pool), dev(case.state_pool)
    y = torch.empty((T, d.num_v_heads * d.head_dim_v), dtype=ydt, device="cuda")
    ws = torch.empty(gdn.gdn_prefill_fused_workspace_bytes(d, T, case.num_reqs), dtype=torch.uint8,
                     device="cuda")
    gdn.gdn_prefill_fused(d, dev(case.x_qkv), dev(case.z), dev(case.a), dev(case.b),
                          dev(case.conv_w), dev(case.gamma), pool, state, dev(case.qsl),
                          dev(case.slot_ids), dev(case.has_initial), y, ws, l2_eps=L2_EPS,
                          norm_eps=NORM_EPS, snap_slot_ids=dev(snaps), snap_interval=interval)
    torch.cuda.synchronize()
    d = case.dims
    z = f64(case.z).reshape(T, d.num_v_heads, d.head_dim_v)
    ref = oracle.prefill_snapshots(f64(case.x_qkv), z, f64(case.a), f64(case.b), f64(case.conv_w),
                                   f64(case.gamma), f64(case.conv_pool), f64(case.state_pool),
                                   case.qsl.numpy(), case.slot_ids.numpy(), case.has_initial.numpy(),
                                   snaps.numpy(), interval, d.num_k_heads, d.num_v_heads,
                                   d.head_dim_k, d.head_dim_v, L2_EPS, NORM_EPS)
    return (y, pool, state), ref


def written(case, snaps, interval):
    lens = np.diff(case.qsl.numpy())
    return sorted(int(snaps[r, j]) for r in range(case.num_reqs)
                  for j in range(min(lens[r] // interval, snaps.shape[1])))


@pytest.mark.parametrize("which", ["d128_group", "d128_group_f32y", "d128_rows", "d16_seq"])
def test_prefill_snapshots_parity(which):
    case, snaps, interval = snap_case(which)
    assert gdn.gdn_validate_snapshot_metadata(case.qsl, case.slot_ids, snaps, interval,
                                              case.num_tokens, case.num_slots) == 0
    (y, pool, state), (y_ref, o_ref, hist_ref, st_ref) = run(case, snaps, interval,
                                                             f32y=which.endswith("f32y"))
    used = sorted(int(s) for s in case.slot_ids)
    ws = written(case, snaps, interval)
    assert ws, "the case must take snapshots"
    e_y = rel_l2(f64(y), y_ref)
    e_f = rel_l2(f64(state)[used], st_ref[used])
    e_s = rel_l2(f64(state)[ws], st_ref[ws])
    print(f"{which}: y {e_y:.2e} final states {e_f:.2e} snapshots {e_s:.2e} ({len(ws)})")
    assert e_y <= OUT_TOL and e_f <= STATE_TOL and e_s <= STATE_TOL
    gb = bits(pool)
    for s in ws + used:
        np.testing.assert_array_equal(gb[s], bits(torch.from_numpy(hist_ref[s]).to(case.conv_pool.dtype)),
                                      err_msg=f"history slot {s}")
    rest = sorted(set(range(case.num_slots)) - set(ws) - set(used))
    np.testing.assert_array_equal(gb[rest], bits(case.conv_pool)[rest])
    np.testing.assert_array_equal(bits(state)[rest], bits(case.state_pool)[rest])


@pytest.mark.parametrize("f32y", [False, True])
def test_prefill_snapshots_bf16_state(f32y):
    """A bf16 state with snapshots: whole-head blocks (bf16 y) and key-head
    group blocks (fp32 y)."""
    case, snaps, interval = snap_case("d128_group")
    case.state_pool = case.state_pool.to(torch.bfloat16)
    (y, pool, state), (y_ref, o_ref, hist_ref, st_ref) = run(case, snaps, interval, f32y=f32y)
    assert rel_l2(f64(y), y_ref) <= OUT_TOL
    ws = written(case, snaps, interval)
    used = sorted(int(s) for s in case.slot_ids)
    check_bf16_state(state, st_ref, ws + used, 1e-2, abs_rel=3e-5)
    rest = sorted(set(range(case.num_slots)) - set(ws) - set(used))
    np.testing.assert_array_equal(bits(state)[rest], bits(case.state_pool)[rest])
