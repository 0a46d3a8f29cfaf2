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

OUT_TOL = 2e-3
STATE_TOL = 1e-3
FP32_TOL = 1e-5


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
