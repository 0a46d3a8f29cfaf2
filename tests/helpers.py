"""Shared test utilities: tensor movement, error metrics, oracle glue.

Tolerances for GPU-vs-oracle parity (the oracle is fp64):
  OUT_TOL    rel-L2 of per-token outputs o (and of y = gated norm of o)
  STATE_TOL  rel-L2 of final recurrent states
  FP32_TOL   rel-L2 for single-pass fp32 stages (conv, norms, fp32 GEMM):
             a few fp32 roundings per element, far below the bf16 budget.
Conv history and slot placement are copies and compared bit for bit.
"""
import numpy as np
import torch

import oracle

OUT_TOL = 2e-3
STATE_TOL = 1e-3
FP32_TOL = 1e-5

# Per-row bounds, a row being one (token, value head) of d_v elements.
# The chunked prefill's contractions split each operand into bf16 hi + lo and
# accumulate in fp32: an element's error is absolute, about 1e-5 of the
# output's overall rms (7e-6 rel-L2 measured), not relative to its own row.
# A row of o is therefore held to
#     |do_row| <= O_ROW_REL |o_row| + O_ROW_ABS rms(o) sqrt(d_v)
# (30x the measured absolute level).  y = o / sqrt(mean(o^2) + eps) * w with
# w = gamma * SiLU(z), |SiLU(z)| <= |z|: a perturbation of o_row moves the
# normalised row by at most 2 sqrt(d_v) |do_row| / |o_row|, and the bf16
# rounding of y by at most 2^-9 per element, so
#     |dy_row| <= 2^-8 |y_row| + 2 sqrt(d_v) max|w_row| |do_row|_bound / |o_row|.
O_ROW_REL = 1e-3
O_ROW_ABS = 3e-4


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def bits(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    raise TypeError(t.dtype)


def dev(t, device="cuda"):
    return t.to(device).contiguous()


def bf16_ulp_ok(got, ref_f64, ulps=1):
    """A bf16 output rounded once from a value accurate to fp32 noise: every
    element within `ulps` bf16 ulps of the fp64 reference, plus an absolute
    allowance of 1e-5 x rms(ref) for elements near zero, where fp32 rounding
    of the accumulation (absolute, not relative) decides the bf16 rounding."""
    ref = np.asarray(ref_f64, np.float64)
    g = got.detach().cpu().to(torch.float64).numpy()
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    allowed = ulps * 2.0 ** -7 * np.abs(ref) + 1e-5 * rms
    return bool(np.all(np.abs(g - ref) <= allowed))


def row_norms(x, d):
    x = np.asarray(x, np.float64).reshape(-1, d)
    return np.linalg.norm(x, axis=1)


def o_row_bound(o_ref, d):
    """Allowed |do| per row of o (see O_ROW_REL, O_ROW_ABS)."""
    o_ref = np.asarray(o_ref, np.float64)
    rms = float(np.sqrt(np.mean(o_ref * o_ref))) if o_ref.size else 0.0
    return O_ROW_REL * row_norms(o_ref, d) + O_ROW_ABS * rms * np.sqrt(d)


def check_o_rows(o, o_ref, d):
    """Every row of o within its bound; returns the worst err / bound ratio."""
    err = row_norms(np.asarray(o, np.float64) - o_ref, d)
    bound = o_row_bound(o_ref, d)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    assert ratio <= 1.0, f"o row error {ratio:.2f} x its bound"
    return ratio


def check_y_rows(y, y_ref, o_ref, z, gamma, d):
    """Every row of the gated-norm output y within the bound the o-row bound
    implies (see O_ROW_REL, O_ROW_ABS); rows whose o is exactly zero must give
    y exactly zero.  Returns the worst err / bound ratio."""
    y = np.asarray(y, np.float64).reshape(-1, d)
    y_ref = np.asarray(y_ref, np.float64).reshape(-1, d)
    on = row_norms(o_ref, d)
    wmax = float(np.max(np.abs(gamma))) * np.max(np.abs(np.asarray(z, np.float64).reshape(-1, d)), axis=1)
    err = np.linalg.norm(y - y_ref, axis=1)
    zero = on == 0
    assert not np.any(err[zero] != 0), "a row with o = 0 must give y = 0"
    ob = o_row_bound(o_ref, d)
    with np.errstate(divide="ignore", invalid="ignore"):
        bound = 2.0 ** -8 * np.linalg.norm(y_ref, axis=1) + 2 * np.sqrt(d) * wmax * ob / on
        ratio = np.where(zero, 0.0, err / bound)
    worst = float(np.max(ratio)) if ratio.size else 0.0
    assert worst <= 1.0, f"y row error {worst:.2f} x its bound"
    return worst


def ulp_diff(got_bits, ref_bits):
    """bf16 ulps between two bit patterns of equal sign handling (sign-magnitude
    mapped onto a monotonic integer line)."""
    def mono(b):
        b = b.astype(np.int64) & 0xFFFF
        m = b & 0x7FFF
        return np.where(b & 0x8000, -m, m)
    return np.abs(mono(got_bits) - mono(ref_bits))


def check_bf16_state(got, ref_f64, slots, max_mismatch, abs_rel=1e-6):
    """Stored bf16 states of `slots` against the rounded oracle states: within
    one ulp, except that elements whose exact value nearly cancels (|x| far
    below the state's rms) may be off by the GPU's absolute arithmetic error,
    abs_rel x rms, which can be many ulps of a tiny number."""
    ref = ref_f64[slots]
    g = bits(got)[slots]
    r = bits(torch.from_numpy(oracle.round_bf16(ref)).to(torch.bfloat16))
    d = ulp_diff(g, r)
    gv = f64(got)[slots]
    rms = float(np.sqrt(np.mean(ref * ref)))
    near_zero_ok = np.abs(gv - ref) <= abs_rel * rms + 2.0 ** -8 * np.abs(ref)
    frac = float(np.mean(d != 0))
    bad = (d > 1) & ~near_zero_ok
    print(f"bf16 state: {frac:.2e} of elements differ, {int(np.sum(d > 1))} by > 1 ulp "
          f"(largest |x| among them {float(np.max(np.abs(ref[d > 1]), initial=0.0)):.2e}, rms {rms:.2e})")
    assert not bad.any() and frac <= max_mismatch
