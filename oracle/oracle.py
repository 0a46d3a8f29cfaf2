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
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the C core's parallel region uses (OMP_NUM_THREADS)."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the C core's later parallel regions."""
    _load().oracle_set_num_threads(int(n))


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


def round_bf16(x):
    """Round to the nearest bfloat16 value, ties to even (the state-dtype
    variant stores S in bf16: the engine's `auto` state dtype may resolve away
    from float32, tutorial page, section 01 data-structure table, state row).

    bf16 has float32's exponent range and 8 significant bits: a value is rounded
    to a multiple of 2^(e-7) for 2^e <= |x| < 2^(e+1), e >= -126, and to a
    multiple of 2^-133 below 2^-126 (subnormals); magnitudes that round past
    the largest finite bf16 become infinite.  NaN stays NaN.  Returns float64
    holding the bf16 values exactly."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    ax = np.abs(x[fin])
    e = np.floor(np.log2(ax))
    # log2 can be off by one next to powers of two: fix e so 2^e <= |x| < 2^(e+1)
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    q = np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))  # the quantum
    r = np.rint(x[fin] / q) * q  # np.rint: round half to even
    top = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > top, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


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


def spec_verify(x_qkv, z, a, b, conv_w, gamma, hist_pool, state_pool, qsl, slot_ids,
                spec_slots, has_initial, Hk, Hv, dk, dv, l2_eps, norm_eps):
    """Speculative multi-token verify of the GDN core.

    Each request brings a few tokens at once (the last accepted token followed
    by draft tokens); they pass through conv -> L2 norm -> gated delta rule ->
    gated norm exactly as a prefill of those tokens would.  In addition the
    recurrent state and the conv history reached after EVERY token j are kept,
    in slot spec_slots[r, j] of the state and history pools, so that rejecting
    the drafts after token j rolls the request back to that slot.  The pages
    give this bookkeeping only as extra speculative slots: the tutorial page's
    data-structure table counts extra speculative slots for the conv history,
    and the dispatch page (step 5) passes num_spec into the state-shape
    calculator; the per-position slots are the reading taken.

    Definition used here: the state (history) at position j is that of the same
    request run over its first j + 1 tokens only — each prefix is a separate
    call of conv1d_silu / gated_delta_rule from the request's input slot.

    x_qkv [T, Cqkv], z [T, Hv, dv], a, b [T, Hv]; spec_slots [nreq, max_tokens]
    int; request r has qsl[r+1] - qsl[r] <= max_tokens tokens.  The input slot
    slot_ids[r] is read and left unchanged unless spec_slots[r, 0] names it.
    Returns (y [T, Hv*dv], o [T, Hv, dv], new_hist_pool, new_state_pool).
    """
    x_qkv = _f64(x_qkv)
    hist_pool = _f64(hist_pool)
    state_pool = _f64(state_pool)
    a = _f64(a)
    b = _f64(b)
    T = x_qkv.shape[0]
    slot_ids = np.asarray(slot_ids, np.int64)
    nreq = slot_ids.size
    spec = np.asarray(spec_slots, np.int64).reshape(nreq, -1)
    max_tokens = spec.shape[1]
    qsl = np.asarray(qsl, np.int64)
    lens = np.diff(qsl)
    _check_meta(qsl, slot_ids, T, state_pool.shape[0])
    if np.any(lens > max_tokens):
        raise ValueError("a request has more tokens than spec slots")
    hi = (np.ones(nreq, np.uint8) if has_initial is None
          else np.asarray(has_initial, np.uint8))
    written = [int(spec[r, j]) for r in range(nreq) for j in range(lens[r])]
    if any(s < 0 or s >= state_pool.shape[0] for s in written):
        raise ValueError("spec slot out of range")
    if len(set(written)) != len(written):
        raise ValueError("spec slots must be distinct")
    for r in range(nreq):
        for r2 in range(nreq):
            for j in range(lens[r2]):
                if spec[r2, j] == slot_ids[r] and not (r2 == r and j == 0):
                    raise ValueError("a spec slot may name an input slot only at its own position 0")

    # the outputs do not depend on where the states are kept
    q, k, v, _ = conv1d_update(x_qkv, conv_w, hist_pool, qsl, slot_ids, hi, Hk, Hv, dk, dv,
                               l2_eps)
    o, _ = gated_delta_rule(q, k, v, a, b, state_pool, qsl, slot_ids, hi)
    y = gated_norm(o, z, gamma, norm_eps)

    new_hist = hist_pool.copy()
    new_state = state_pool.copy()
    for j in range(max_tokens):
        sel = [r for r in range(nreq) if lens[r] > j]
        if not sel:
            break
        # every selected request cut to its first j + 1 tokens, in a compact
        # pool of its own input slots
        rows = np.concatenate([np.arange(qsl[r], qsl[r] + j + 1) for r in sel])
        sub_qsl = np.arange(len(sel) + 1) * (j + 1)
        sub_slots = np.arange(len(sel))
        sub_hi = hi[sel]
        _, hist_j = conv1d_silu(x_qkv[rows], conv_w, hist_pool[slot_ids[sel]], sub_qsl,
                                sub_slots, sub_hi)
        _, st_j = gated_delta_rule(q[rows], k[rows], v[rows], a[rows], b[rows],
                                   state_pool[slot_ids[sel]], sub_qsl, sub_slots, sub_hi)
        for i, r in enumerate(sel):
            new_hist[spec[r, j]] = hist_j[i]
            new_state[spec[r, j]] = st_j[i]
    return y, o, new_hist, new_state


def prefill_snapshots(x_qkv, z, a, b, conv_w, gamma, hist_pool, state_pool, qsl, slot_ids,
                      has_initial, snap_slots, interval, Hk, Hv, dk, dv, l2_eps, norm_eps):
    """A prefill that also keeps prefix-cache snapshots ("align" mode).

    The dispatch page shows the hybrid model refusing prefix caching in mode
    'all' and asking for '--mamba-cache-mode=align' instead; the pages say no
    more.  Reading taken: in align mode the prefill keeps, besides the final
    state, the recurrent state and conv history reached after every
    `interval` tokens of the call, so that a later request sharing that
    prefix can start from them.  Snapshot j of request r (for
    (j + 1) * interval <= its length, and j < snap_slots.shape[1]) is the state
    and history after its first (j + 1) * interval tokens, written to slot
    snap_slots[r, j] of both pools.

    Definition used here: each snapshot is a separate prefill of the prefix
    from the request's input slot (conv1d_silu / gated_delta_rule on the
    first (j + 1) * interval tokens); the outputs and the final state and
    history are those of the whole request.
    Returns (y [T, Hv*dv], o [T, Hv, dv], new_hist_pool, new_state_pool).
    """
    x_qkv = _f64(x_qkv)
    hist_pool = _f64(hist_pool)
    state_pool = _f64(state_pool)
    a = _f64(a)
    b = _f64(b)
    T = x_qkv.shape[0]
    slot_ids = np.asarray(slot_ids, np.int64)
    nreq = slot_ids.size
    snaps = np.asarray(snap_slots, np.int64).reshape(nreq, -1)
    max_snaps = snaps.shape[1]
    qsl = np.asarray(qsl, np.int64)
    lens = np.diff(qsl)
    _check_meta(qsl, slot_ids, T, state_pool.shape[0])
    if interval <= 0:
        raise ValueError("snapshot interval must be positive")
    hi = (np.ones(nreq, np.uint8) if has_initial is None
          else np.asarray(has_initial, np.uint8))
    nsnap = [int(min(lens[r] // interval, max_snaps)) for r in range(nreq)]
    written = [int(snaps[r, j]) for r in range(nreq) for j in range(nsnap[r])]
    if any(s_ < 0 or s_ >= state_pool.shape[0] for s_ in written):
        raise ValueError("snapshot slot out of range")
    if len(set(written)) != len(written) or set(written) & set(int(s_) for s_ in slot_ids):
        raise ValueError("snapshot slots must be distinct from each other and from the requests' slots")

    q, k, v, new_hist = conv1d_update(x_qkv, conv_w, hist_pool, qsl, slot_ids, hi, Hk, Hv, dk,
                                      dv, l2_eps)
    o, new_state = gated_delta_rule(q, k, v, a, b, state_pool, qsl, slot_ids, hi)
    y = gated_norm(o, z, gamma, norm_eps)
    for j in range(max_snaps):
        sel = [r for r in range(nreq) if nsnap[r] > j]
        if not sel:
            break
        n = (j + 1) * interval
        rows = np.concatenate([np.arange(qsl[r], qsl[r] + n) for r in sel])
        sub_qsl = np.arange(len(sel) + 1) * n
        sub_slots = np.arange(len(sel))
        _, hist_j = conv1d_silu(x_qkv[rows], conv_w, hist_pool[slot_ids[sel]], sub_qsl, sub_slots,
                                hi[sel])
        _, st_j = gated_delta_rule(q[rows], k[rows], v[rows], a[rows], b[rows],
                                   state_pool[slot_ids[sel]], sub_qsl, sub_slots, hi[sel])
        for i, r in enumerate(sel):
            new_hist[snaps[r, j]] = hist_j[i]
            new_state[snaps[r, j]] = st_j[i]
    return y, o, new_hist, new_state


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
