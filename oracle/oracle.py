"""fp64 CPU oracle of the Gated DeltaNet mixer core — TEST INFRASTRUCTURE ONLY.

Every function takes and returns float64 numpy arrays holding the exact values
the GPU received (bf16 inputs are widened exactly).  The recurrence runs in the
C core ``gdn_oracle.c`` (sequential in time, OpenMP across independent
(request, value head) units); everything else is written here in numpy.

Citations name the page "Qwen3.8-27B: from model structure to the vLLM
inference dataflow" (below: the tutorial page) and the page "How the 64 layers
of Qwen3.8-27B are dispatched in vLLM" (below: the dispatch page).

Readings taken where the pages are silent (each one is listed in the design
notes with its reason):
  * alpha = exp(-softplus(a)), beta = sigmoid(b): the pages only name the raw
    projections a and b.
  * conv weight w[c, i] multiplies the input i steps back; no bias.
  * history is stored oldest -> newest: hist[c, 0] = x[t-3] ... hist[c, 2] = x[t-1].
  * L2-norm and RMSNorm epsilons sit inside the square root.
  * the gated RMSNorm normalises each value head over d_v with one shared gain.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        up = ctypes.POINTER(ctypes.c_uint8)
        lib.oracle_gdn_recurrence.argtypes = [
            ctypes.c_int32, ip, ip, up, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_gdn_recurrence.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the C core's parallel region uses (OMP_NUM_THREADS)."""
    return int(_load().oracle_num_threads())


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _check_meta(qsl, slot_ids, num_tokens, num_slots):
    qsl = np.asarray(qsl)
    slot_ids = np.asarray(slot_ids)
    if qsl.ndim != 1 or qsl.size != slot_ids.size + 1:
        raise ValueError("query_start_loc must have num_reqs + 1 entries")
    if qsl.size and (qsl[0] != 0 or qsl[-1] != num_tokens):
        raise ValueError("query_start_loc must start at 0 and end at T")
    if np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc must be non-decreasing")
    if slot_ids.size and (slot_ids.min() < 0 or slot_ids.max() >= num_slots):
        raise ValueError("slot id out of range")
    if np.unique(slot_ids).size != slot_ids.size:
        raise ValueError("slot ids must be distinct")


# ---------------------------------------------------------------------------
# elementwise maps (textbook definitions)
# ---------------------------------------------------------------------------
def silu(y):
    """SiLU(y) = y * sigmoid(y) (tutorial page, section 01 operator table)."""
    y = _f64(y)
    return y / (1.0 + np.exp(-y))


def gates(a, b):
    """alpha = exp(-softplus(a)), beta = sigmoid(b).

    The tutorial page (section 01 operator table, in-projection row) names only
    the raw projections a, b of shape [T, 48]; this mapping is the reading
    taken, with softplus(x) = log(1 + e^x) (numpy's logaddexp(0, x)).
    """
    a = _f64(a)
    b = _f64(b)
    alpha = np.exp(-np.logaddexp(0.0, a))
    beta = 1.0 / (1.0 + np.exp(-b))
    return alpha, beta


def l2norm(x, eps):
    """x / sqrt(sum(x^2) + eps) over the last axis (operator table, conv row:
    q = normalize(q), k = normalize(k))."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def rmsnorm(x, gamma, eps):
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis (operator table,
    first row; the tutorial page's final-norm worked example fixes RMS, not
    LayerNorm, normalisation)."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(gamma)


def gated_norm(o, z, gamma, eps):
    """Ogate = RMSNorm(o) * SiLU(Z) (operator table, gated-output row).

    o, z: [T, Hv, dv]; the RMS is taken per (token, value head) over dv with a
    gain gamma [dv] shared by all heads.  Returns y [T, Hv * dv].
    """
    o = _f64(o)
    z = _f64(z)
    y = rmsnorm(o, gamma, eps) * silu(z)
    return y.reshape(o.shape[0], -1)


def linear(x, w):
    """x @ w (a library fp64 matrix product)."""
    return _f64(x) @ _f64(w)


def residual_add(x, delta):
    """Y = X + Delta_mix (operator table, residual row)."""
    return _f64(x) + _f64(delta)


# ---------------------------------------------------------------------------
# causal depthwise conv1d + SiLU with per-request history
# ---------------------------------------------------------------------------
def conv1d_silu(x, conv_w, hist_pool, qsl, slot_ids, has_initial=None):
    """c_t = SiLU(sum_{i=0}^{taps-1} w_i * x_{t-i}) per channel (operator table,
    conv row; data-structure table, conv history row: 3 past inputs are kept,
    the 4-tap window includes the current one).

    x         [T, C]             the request-packed conv input
    conv_w    [C, taps]          conv_w[c, i] multiplies x[t - i]
    hist_pool [slots, C, taps-1] oldest -> newest history per slot
    Returns (c [T, C], new_hist_pool).  A request reads only its own history
    (zeros when has_initial is 0), never the previous request's rows; its new
    history is the last taps-1 entries of [history, own rows].  Empty requests
    leave their slot untouched.
    """
    x = _f64(x)
    w = _f64(conv_w)
    hist_pool = _f64(hist_pool)
    T, C = x.shape
    taps = w.shape[1]
    nh = taps - 1
    nreq = len(slot_ids)
    _check_meta(qsl, slot_ids, T, hist_pool.shape[0])
    if has_initial is None:
        has_initial = np.ones(nreq, dtype=np.uint8)
    out = np.zeros((T, C))
    new_pool = hist_pool.copy()
    for r in range(nreq):
        t0, t1 = int(qsl[r]), int(qsl[r + 1])
        if t1 == t0:
            continue
        s = int(slot_ids[r])
        hist = hist_pool[s].T if has_initial[r] else np.zeros((nh, C))  # [nh, C]
        window = np.concatenate([hist, x[t0:t1]], axis=0)  # [nh + L, C]
        L = t1 - t0
        y = np.zeros((L, C))
        for i in range(taps):
            # x_{t-i} for t = 0..L-1 sits at window row nh + t - i
            y += w[:, i] * window[nh - i: nh - i + L]
        out[t0:t1] = silu(y)
        new_pool[s] = window[-nh:].T
    return out, new_pool


def split_qkv(c, Hk, Hv, dk, dv):
    """Split conv output [T, 2*Hk*dk + Hv*dv] into q [T,Hk,dk], k [T,Hk,dk],
    v [T,Hv,dv] in the Q0, K0, V0 order of the in-projection row."""
    c = _f64(c)
    T = c.shape[0]
    nq = Hk * dk
    q = c[:, :nq].reshape(T, Hk, dk)
    k = c[:, nq:2 * nq].reshape(T, Hk, dk)
    v = c[:, 2 * nq:2 * nq + Hv * dv].reshape(T, Hv, dv)
    return q, k, v


def conv1d_update(x, conv_w, hist_pool, qsl, slot_ids, has_initial, Hk, Hv, dk,
                  dv, l2_eps):
    """conv1d + SiLU, then L2-normalised q, k; v unnormalised.
    Returns (q, k, v, new_hist_pool)."""
    c, new_pool = conv1d_silu(x, conv_w, hist_pool, qsl, slot_ids, has_initial)
    q, k, v = split_qkv(c, Hk, Hv, dk, dv)
    return l2norm(q, l2_eps), l2norm(k, l2_eps), v.copy(), new_pool


# ---------------------------------------------------------------------------
# gated delta rule (C core)
# ---------------------------------------------------------------------------
def gated_delta_rule(q, k, v, a, b, state_pool, qsl, slot_ids, has_initial=None):
    """Sequential gated delta rule over a packed batch (operator table, GDN row;
    GDN state lab; evidence matrix row on decaying before reading the error).

    q, k [T,Hk,dk]; v [T,Hv,dv]; a, b [T,Hv] raw; state_pool [slots,Hv,dv,dk].
    Returns (o [T,Hv,dv], new_state_pool).  The state shape depends only on
    heads and dims, never on T (dispatch page, step 5: the state-shape
    calculator takes no sequence length).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    T, Hk, dk = q.shape
    _, Hv, dv = v.shape
    if k.shape != q.shape or v.shape[0] != T or Hv % Hk:
        raise ValueError("inconsistent q/k/v shapes")
    alpha, beta = gates(a, b)
    alpha = _f64(alpha.reshape(T, Hv))
    beta = _f64(beta.reshape(T, Hv))
    pool = _f64(state_pool).copy()
    if pool.shape[1:] != (Hv, dv, dk):
        raise ValueError("state pool must be [slots, Hv, dv, dk]")
    nreq = len(slot_ids)
    _check_meta(qsl, slot_ids, T, pool.shape[0])
    qsl_a = _i32(qsl)
    slot_a = _i32(slot_ids)
    hi = np.ascontiguousarray(
        np.ones(nreq, np.uint8) if has_initial is None else np.asarray(has_initial, np.uint8))
    o = np.zeros((T, Hv, dv))
    lib = _load()
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    up = ctypes.POINTER(ctypes.c_uint8)
    rc = lib.oracle_gdn_recurrence(
        nreq, qsl_a.ctypes.data_as(ip), slot_a.ctypes.data_as(ip),
        hi.ctypes.data_as(up), Hk, Hv, dk, dv, q.ctypes.data_as(dp),
        k.ctypes.data_as(dp), v.ctypes.data_as(dp), alpha.ctypes.data_as(dp),
        beta.ctypes.data_as(dp), pool.ctypes.data_as(dp), o.ctypes.data_as(dp))
    if rc != 0:
        raise MemoryError("oracle recurrence failed to allocate")
    return o, pool


def decode_step(q, k, v, a, b, state_pool, slot_ids):
    """One token per request: the same recurrence with every request of length
    1 continuing its slot's state (tutorial page, section 02: decode advances
    each active sequence by one token per step)."""
    R = len(slot_ids)
    qsl = np.arange(R + 1, dtype=np.int32)
    return gated_delta_rule(q, k, v, a, b, state_pool, qsl, slot_ids,
                            np.ones(R, np.uint8))


# ---------------------------------------------------------------------------
# one GDN layer block (operator table rows 1-8)
# ---------------------------------------------------------------------------
def gdn_layer(X, gamma_in, W_qkvz, W_ba, conv_w, gamma_out, W_o, hist_pool,
              state_pool, qsl, slot_ids, has_initial, Hk, Hv, dk, dv,
              norm_eps, l2_eps):
    """X -> RMSNorm -> [Q0,K0,V0,Z] = U Wqkvz, [b, a] = U Wba -> conv1d+SiLU ->
    L2 norm -> gated delta rule -> RMSNorm(o) * SiLU(Z) -> Wo -> + X.

    W_qkvz [hidden, 2*Hk*dk + 2*Hv*dv] stacks q | k | v | z columns and W_ba
    [hidden, 2*Hv] stacks b | a (dispatch page, step 7: in_proj_qkv/z stack into
    in_proj_qkvz at (0,1,2) and 3; in_proj_b/a stack into in_proj_ba at 0 and 1).
    Returns (Y, new_hist_pool, new_state_pool, intermediates dict).
    """
    T = X.shape[0]
    U = rmsnorm(X, gamma_in, norm_eps)
    P = linear(U, W_qkvz)
    BA = linear(U, W_ba)
    cq = 2 * Hk * dk + Hv * dv
    x_qkv = P[:, :cq]
    Z = P[:, cq:].reshape(T, Hv, dv)
    b = BA[:, :Hv]
    a = BA[:, Hv:]
    q, k, v, new_hist = conv1d_update(x_qkv, conv_w, hist_pool, qsl, slot_ids,
                                      has_initial, Hk, Hv, dk, dv, l2_eps)
    o, new_state = gated_delta_rule(q, k, v, a, b, state_pool, qsl, slot_ids,
                                    has_initial)
    y = gated_norm(o, Z, gamma_out, norm_eps)
    Y = residual_add(X, linear(y, W_o))
    inter = dict(U=U, x_qkv=x_qkv, Z=Z, a=a, b=b, q=q, k=k, v=v, o=o, y=y)
    return Y, new_hist, new_state, inter
