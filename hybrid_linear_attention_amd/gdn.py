"""Thin ctypes binding of libgdn (include/gdn.h).

Every function has the name of the C entry point it calls and only marshals
arguments: torch tensors (device memory) become raw pointers, dtypes become
``gdn_dtype`` codes, and the current torch stream becomes the ``hipStream_t``.
No arithmetic of the method happens here.  A missing library, a CPU tensor or a
non-OK status raises; there is no fallback path.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
GDN_FP8_E4M3 = 2
GDN_NOALLOC_SCRATCH_BYTES = 256 << 20  # include/gdn.h: the static scratch of gdn_prefill_fused_noalloc

STATUS = {
    0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_DIMS", 3: "GDN_ERR_DTYPE",
    4: "GDN_ERR_SHAPE", 5: "GDN_ERR_WORKSPACE", 6: "GDN_ERR_ALIGN", 7: "GDN_ERR_HIP",
    8: "GDN_ERR_METADATA", 9: "GDN_ERR_SCRATCH",
}


class GdnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class GdnDimsC(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("conv_taps", ctypes.c_int32)]


class GqaDimsC(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rotary_dim", ctypes.c_int32)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_SIGS = {
    "gdn_status_string": ([_i32], ctypes.c_char_p),
    "gdn_version": ([], ctypes.c_char_p),
    "gdn_conv1d_update": ([ctypes.POINTER(GdnDimsC), _vp, _i32, _i64, _vp, _i32, _vp, _i32, _vp,
                           _vp, _vp, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _i32, _vp], _i32),
    "gdn_decode_step": ([ctypes.POINTER(GdnDimsC), _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64, _vp,
                         _vp, _i32, _i32, _vp, _i32, _vp], _i32),
    "gdn_decode_fused": ([ctypes.POINTER(GdnDimsC), _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i32, _vp,
                          _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _f32, _f32, _vp, _i32,
                          _vp, _vp], _i32),
    "gdn_spec_verify": ([ctypes.POINTER(GdnDimsC), _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i32, _vp,
                         _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                         _f32, _f32, _vp, _i32, _vp, _vp], _i32),
    "gdn_prefill_workspace_bytes": ([ctypes.POINTER(GdnDimsC), _i32, _i32], ctypes.c_size_t),
    "gdn_prefill_fused_workspace_bytes": ([ctypes.POINTER(GdnDimsC), _i32, _i32], ctypes.c_size_t),
    "gdn_prefill_fused": ([ctypes.POINTER(GdnDimsC), _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i32, _vp,
                           _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32,
                           _i32, _f32, _f32, _vp, _i32, _vp, ctypes.c_size_t, _vp], _i32),
    "gdn_prefill_fused_noalloc": ([ctypes.POINTER(GdnDimsC), _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i32,
                                   _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                                   _vp, _i32, _i32, _f32, _f32, _vp, _i32, _vp], _i32),
    "gdn_prefill_varlen": ([ctypes.POINTER(GdnDimsC), _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i64,
                            _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, ctypes.c_size_t,
                            _vp], _i32),
    "gdn_gated_norm": ([ctypes.POINTER(GdnDimsC), _vp, _i32, _vp, _i32, _i64, _vp, _i32, _f32, _i32,
                        _vp, _i32, _vp], _i32),
    "gdn_rmsnorm": ([_vp, _i32, _vp, _i32, _f32, _i32, _i32, _vp, _i32, _vp], _i32),
    "gdn_gemm_bf16": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _i32, _i32, _vp], _i32),
    "gdn_gemm_bf16_ws": ([_vp, _i64, _vp, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _i32, _i32, _vp,
                          ctypes.c_size_t, _vp], _i32),
    "gdn_gemm_bf16_workspace_bytes": ([_i32, _i32, _i32], ctypes.c_size_t),
    "gdn_validate_metadata": ([_vp, _vp, _i32, _i32, _i32], _i32),
    "gdn_validate_spec_metadata": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32], _i32),
    "gdn_validate_snapshot_metadata": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32], _i32),
    "gqa_decode_workspace_bytes": ([ctypes.POINTER(GqaDimsC), _i32, _i32], ctypes.c_size_t),
    "gqa_decode_paged": ([ctypes.POINTER(GqaDimsC), _vp, _i64, _vp, _i64, _vp, _vp, _i64, _i32, _vp,
                          _vp, _i32, _f32, _f32, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                          ctypes.c_double, _vp, _i32, _vp, _vp, ctypes.c_size_t, _vp], _i32),
    "gqa_validate_decode_metadata": ([_vp, _i32, _vp, _i32, _i32, _i32, _i32], _i32),
}

SPEC_MAX_TOKENS = 8

_lib = None


def lib():
    """The loaded libgdn (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m hybrid_linear_attention_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (argtypes, restype) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = handle
    return _lib


def dims_c(dims) -> GdnDimsC:
    if isinstance(dims, GdnDimsC):
        return dims
    if isinstance(dims, (tuple, list)):
        return GdnDimsC(*[int(x) for x in dims])
    return GdnDimsC(int(dims.num_k_heads), int(dims.num_v_heads), int(dims.head_dim_k),
                    int(dims.head_dim_v), int(dims.conv_taps))


def _dt(t):
    if t.dtype == torch.float32:
        return GDN_F32
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, what=""):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor must live on the GPU")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _rows(t, what):
    """Leading dimension of a 2-D (or flattened) row-major view."""
    if t.stride(-1) != 1:
        raise ValueError(f"{what}: innermost dimension must be contiguous")
    return t.stride(0)


def _check(status, where):
    if status != 0:
        raise GdnError(status, where)


def _contig(t, what):
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    return t


def gdn_conv1d_update(dims, x, conv_w, conv_pool, query_start_loc, slot_ids, has_initial,
                      q, k, v, l2_eps=1e-6, stream=None):
    """x [T, >=Cqkv] (row stride = x_ld); outputs q, k [T,Hk,dk], v [T,Hv,dv]."""
    d = dims_c(dims)
    for name, t in (("conv_w", conv_w), ("conv_pool", conv_pool), ("q", q), ("k", k), ("v", v)):
        _contig(t, name)
    st = lib().gdn_conv1d_update(
        ctypes.byref(d), _ptr(x, "x"), _dt(x), _rows(x, "x"), _ptr(conv_w, "conv_w"), _dt(conv_w),
        _ptr(conv_pool, "conv_pool"), _dt(conv_pool), _ptr(query_start_loc, "qsl"),
        _ptr(slot_ids, "slot_ids"), _ptr(has_initial, "has_initial"), slot_ids.numel(),
        x.shape[0], conv_pool.shape[0], float(l2_eps), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"),
        _dt(q), _stream(stream))
    _check(st, "gdn_conv1d_update")


def gdn_decode_step(dims, q, k, v, a, b, state_pool, slot_ids, o, stream=None):
    """One token per request; a, b [R, >=Hv] raw gates (row stride = gate_ld)."""
    d = dims_c(dims)
    if a.stride() != b.stride() or a.dtype != b.dtype:
        raise ValueError("a and b must share dtype and strides")
    for name, t in (("q", q), ("k", k), ("v", v), ("state_pool", state_pool), ("o", o)):
        _contig(t, name)
    if state_pool.dtype != torch.float32:
        raise TypeError("state_pool must be float32")
    st = lib().gdn_decode_step(
        ctypes.byref(d), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _dt(q), _ptr(a, "a"),
        _ptr(b, "b"), _dt(a), _rows(a, "a"), _ptr(state_pool, "state_pool"),
        _ptr(slot_ids, "slot_ids"), slot_ids.numel(), state_pool.shape[0], _ptr(o, "o"), _dt(o),
        _stream(stream))
    _check(st, "gdn_decode_step")


def gdn_decode_fused(dims, x, z, a, b, conv_w, gamma, conv_pool, state_pool, slot_ids, y,
                     has_initial=None, o=None, l2_eps=1e-6, norm_eps=1e-6, stream=None):
    """One decode step (conv update -> recurrence -> gated norm) in one launch.
    x [R, >=Cqkv], z [R, >=Hv*dv], a, b [R, >=Hv] share one dtype and give their
    row strides; state_pool fp32 or bf16 (its dtype is passed as state_dt);
    y [R, Hv*dv]; o optional fp32 [R, Hv, dv]."""
    d = dims_c(dims)
    if a.stride() != b.stride() or not (x.dtype == z.dtype == a.dtype == b.dtype == conv_pool.dtype):
        raise ValueError("x, z, a, b and conv_pool share one dtype; a and b share strides")
    if conv_w.dtype != gamma.dtype:
        raise ValueError("conv_w and gamma share one dtype")
    for name, t in (("conv_w", conv_w), ("gamma", gamma), ("conv_pool", conv_pool),
                    ("state_pool", state_pool), ("y", y)):
        _contig(t, name)
    if o is not None and o.dtype != torch.float32:
        raise TypeError("o must be float32")
    zz = z.reshape(z.shape[0], -1) if z.is_contiguous() else z
    st = lib().gdn_decode_fused(
        ctypes.byref(d), _ptr(x, "x"), _rows(x, "x"), _ptr(zz, "z"), _rows(zz, "z"), _ptr(a, "a"),
        _ptr(b, "b"), _rows(a, "a"), _dt(x), _ptr(conv_w, "conv_w"), _ptr(gamma, "gamma"),
        _dt(conv_w), _ptr(conv_pool, "conv_pool"), _ptr(state_pool, "state_pool"),
        _dt(state_pool), _ptr(slot_ids, "slot_ids"), _ptr(has_initial, "has_initial"), slot_ids.numel(),
        state_pool.shape[0], float(l2_eps), float(norm_eps), _ptr(y, "y"), _dt(y),
        _ptr(o, "o"), _stream(stream))
    _check(st, "gdn_decode_fused")


def gdn_spec_verify(dims, x, z, a, b, conv_w, gamma, conv_pool, state_pool, query_start_loc,
                    slot_ids, spec_slot_ids, y, has_initial=None, o=None, l2_eps=1e-6,
                    norm_eps=1e-6, stream=None):
    """Speculative multi-token verify in one launch.  x [T, >=Cqkv], z [T, >=Hv*dv],
    a, b [T, >=Hv] share one dtype and give their row strides; spec_slot_ids
    int32 [R, max_tokens]; y [T, Hv*dv]; o optional fp32 [T, Hv, dv]."""
    d = dims_c(dims)
    if a.stride() != b.stride() or not (x.dtype == z.dtype == a.dtype == b.dtype == conv_pool.dtype):
        raise ValueError("x, z, a, b and conv_pool share one dtype; a and b share strides")
    if conv_w.dtype != gamma.dtype:
        raise ValueError("conv_w and gamma share one dtype")
    for name, t in (("conv_w", conv_w), ("gamma", gamma), ("conv_pool", conv_pool),
                    ("state_pool", state_pool), ("y", y), ("spec_slot_ids", spec_slot_ids)):
        _contig(t, name)
    if o is not None and o.dtype != torch.float32:
        raise TypeError("o must be float32")
    if spec_slot_ids.dim() != 2 or spec_slot_ids.shape[0] != slot_ids.numel():
        raise ValueError("spec_slot_ids must be [num_reqs, max_tokens]")
    zz = z.reshape(z.shape[0], -1) if z.is_contiguous() else z
    st = lib().gdn_spec_verify(
        ctypes.byref(d), _ptr(x, "x"), _rows(x, "x"), _ptr(zz, "z"), _rows(zz, "z"), _ptr(a, "a"),
        _ptr(b, "b"), _rows(a, "a"), _dt(x), _ptr(conv_w, "conv_w"), _ptr(gamma, "gamma"),
        _dt(conv_w), _ptr(conv_pool, "conv_pool"), _ptr(state_pool, "state_pool"),
        _dt(state_pool), _ptr(query_start_loc, "qsl"), _ptr(slot_ids, "slot_ids"),
        _ptr(spec_slot_ids, "spec_slot_ids"), spec_slot_ids.shape[1],
        _ptr(has_initial, "has_initial"), slot_ids.numel(), x.shape[0], state_pool.shape[0],
        float(l2_eps), float(norm_eps), _ptr(y, "y"), _dt(y), _ptr(o, "o"), _stream(stream))
    _check(st, "gdn_spec_verify")


def gdn_prefill_workspace_bytes(dims, num_tokens, num_reqs):
    d = dims_c(dims)
    return int(lib().gdn_prefill_workspace_bytes(ctypes.byref(d), int(num_tokens), int(num_reqs)))


def gdn_prefill_varlen(dims, q, k, v, a, b, state_pool, query_start_loc, slot_ids, has_initial,
                       o, workspace=None, stream=None):
    """Packed varlen prefill; workspace is a uint8 device tensor of at least
    gdn_prefill_workspace_bytes(...) bytes (may be None when that is 0)."""
    d = dims_c(dims)
    if a.stride() != b.stride() or a.dtype != b.dtype:
        raise ValueError("a and b must share dtype and strides")
    for name, t in (("q", q), ("k", k), ("v", v), ("state_pool", state_pool), ("o", o)):
        _contig(t, name)
    if state_pool.dtype != torch.float32:
        raise TypeError("state_pool must be float32")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = lib().gdn_prefill_varlen(
        ctypes.byref(d), _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _dt(q), _ptr(a, "a"),
        _ptr(b, "b"), _dt(a), _rows(a, "a"), _ptr(state_pool, "state_pool"),
        _ptr(query_start_loc, "qsl"), _ptr(slot_ids, "slot_ids"), _ptr(has_initial, "has_initial"),
        slot_ids.numel(), q.shape[0], state_pool.shape[0], _ptr(o, "o"), _dt(o), ws_ptr, ws_bytes,
        _stream(stream))
    _check(st, "gdn_prefill_varlen")


def gdn_prefill_fused_workspace_bytes(dims, num_tokens, num_reqs):
    d = dims_c(dims)
    return int(lib().gdn_prefill_fused_workspace_bytes(ctypes.byref(d), int(num_tokens),
                                                       int(num_reqs)))


def _prefill_fused_args(dims, x, z, a, b, conv_w, gamma, conv_pool, state_pool, query_start_loc,
                        slot_ids, has_initial, y, l2_eps, norm_eps, snap_slot_ids, snap_interval):
    """The arguments gdn_prefill_fused and gdn_prefill_fused_noalloc share, up to
    and including y_dt, after the binding's own checks."""
    d = dims_c(dims)
    if a.stride() != b.stride() or not (x.dtype == z.dtype == a.dtype == b.dtype == conv_pool.dtype):
        raise ValueError("x, z, a, b and conv_pool share one dtype; a and b share strides")
    if conv_w.dtype != gamma.dtype:
        raise ValueError("conv_w and gamma share one dtype")
    for name, t in (("conv_w", conv_w), ("gamma", gamma), ("conv_pool", conv_pool),
                    ("state_pool", state_pool), ("y", y)):
        _contig(t, name)
    zz = z.reshape(z.shape[0], -1) if z.is_contiguous() else z
    max_snaps = 0
    if snap_slot_ids is not None:
        _contig(snap_slot_ids, "snap_slot_ids")
        if snap_slot_ids.dim() != 2 or snap_slot_ids.shape[0] != slot_ids.numel():
            raise ValueError("snap_slot_ids must be [num_reqs, max_snaps]")
        max_snaps = snap_slot_ids.shape[1]
    return (ctypes.byref(d), _ptr(x, "x"), _rows(x, "x"), _ptr(zz, "z"), _rows(zz, "z"),
            _ptr(a, "a"), _ptr(b, "b"), _rows(a, "a"), _dt(x), _ptr(conv_w, "conv_w"),
            _ptr(gamma, "gamma"), _dt(conv_w), _ptr(conv_pool, "conv_pool"),
            _ptr(state_pool, "state_pool"), _dt(state_pool), _ptr(query_start_loc, "qsl"),
            _ptr(slot_ids, "slot_ids"), _ptr(has_initial, "has_initial"), slot_ids.numel(),
            x.shape[0], state_pool.shape[0], _ptr(snap_slot_ids, "snap_slot_ids"), max_snaps,
            int(snap_interval), float(l2_eps), float(norm_eps), _ptr(y, "y"), _dt(y))


def gdn_prefill_fused(dims, x, z, a, b, conv_w, gamma, conv_pool, state_pool, query_start_loc,
                      slot_ids, has_initial, y, workspace, l2_eps=1e-6, norm_eps=1e-6,
                      snap_slot_ids=None, snap_interval=0, stream=None):
    """A whole prefill step (conv update -> recurrence -> gated norm) over a packed
    batch; x, z, a, b share one dtype and give their row strides; state_pool fp32
    or bf16; y [T, Hv*dv];
    workspace a uint8 device tensor of gdn_prefill_fused_workspace_bytes(...);
    snap_slot_ids int32 [R, max_snaps] with snap_interval (tokens, a multiple of
    32) keeps prefix-cache snapshots."""
    args = _prefill_fused_args(dims, x, z, a, b, conv_w, gamma, conv_pool, state_pool,
                               query_start_loc, slot_ids, has_initial, y, l2_eps, norm_eps,
                               snap_slot_ids, snap_interval)
    st = lib().gdn_prefill_fused(*args, _ptr(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gdn_prefill_fused")


def gdn_prefill_fused_noalloc(dims, x, z, a, b, conv_w, gamma, conv_pool, state_pool,
                              query_start_loc, slot_ids, has_initial, y, l2_eps=1e-6,
                              norm_eps=1e-6, snap_slot_ids=None, snap_interval=0, stream=None):
    """gdn_prefill_fused on the library's static scratch (no workspace, nothing
    allocated); raises GdnError (GDN_ERR_SCRATCH) for a batch larger than it."""
    args = _prefill_fused_args(dims, x, z, a, b, conv_w, gamma, conv_pool, state_pool,
                               query_start_loc, slot_ids, has_initial, y, l2_eps, norm_eps,
                               snap_slot_ids, snap_interval)
    st = lib().gdn_prefill_fused_noalloc(*args, _stream(stream))
    _check(st, "gdn_prefill_fused_noalloc")


def gdn_gated_norm(dims, o, z, gamma, y, eps=1e-6, stream=None):
    """o [T,Hv,dv]; z [T, >=Hv*dv] (row stride = z_ld); gamma [dv]; y [T, Hv*dv]."""
    d = dims_c(dims)
    for name, t in (("o", o), ("gamma", gamma), ("y", y)):
        _contig(t, name)
    zz = z.reshape(z.shape[0], -1) if z.is_contiguous() else z
    st = lib().gdn_gated_norm(
        ctypes.byref(d), _ptr(o, "o"), _dt(o), _ptr(zz, "z"), _dt(zz), _rows(zz, "z"),
        _ptr(gamma, "gamma"), _dt(gamma), float(eps), o.shape[0], _ptr(y, "y"), _dt(y),
        _stream(stream))
    _check(st, "gdn_gated_norm")


def gdn_rmsnorm(x, gamma, y, eps=1e-6, stream=None):
    for name, t in (("x", x), ("gamma", gamma), ("y", y)):
        _contig(t, name)
    st = lib().gdn_rmsnorm(_ptr(x, "x"), _dt(x), _ptr(gamma, "gamma"), _dt(gamma), float(eps),
                           x.shape[0], x.shape[1], _ptr(y, "y"), _dt(y), _stream(stream))
    _check(st, "gdn_rmsnorm")


def gdn_gemm_bf16_workspace_bytes(M, N, K):
    """Workspace bytes gdn_gemm_bf16 can use for this shape on the current device
    (0: it would split nothing)."""
    return int(lib().gdn_gemm_bf16_workspace_bytes(int(M), int(N), int(K)))


def gdn_gemm_bf16(A, B, C, residual=None, stream=None, workspace=None):
    """C[M,N] = A[M,K] @ B[N,K]^T (+ residual); A, B, residual bf16; row strides taken
    from the tensors (innermost dimension contiguous).  With a workspace (uint8
    device tensor of gdn_gemm_bf16_workspace_bytes(M, N, K) bytes) the last,
    partly filled round of tiles is split along K (gdn_gemm_bf16_ws)."""
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or C.shape[0] != M or C.shape[1] != N:
        raise ValueError("gemm shape mismatch")
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    r_ptr, ldr = None, 0
    if residual is not None:
        if residual.dtype != torch.bfloat16 or tuple(residual.shape) != (M, N):
            raise ValueError("residual must be bf16 [M, N]")
        r_ptr, ldr = _ptr(residual, "residual"), _rows(residual, "residual")
    if workspace is None:
        st = lib().gdn_gemm_bf16(_ptr(A, "A"), _rows(A, "A"), _ptr(B, "B"), _rows(B, "B"),
                                 _ptr(C, "C"), _rows(C, "C"), _dt(C), r_ptr, ldr, M, N, K,
                                 _stream(stream))
        _check(st, "gdn_gemm_bf16")
        return
    st = lib().gdn_gemm_bf16_ws(_ptr(A, "A"), _rows(A, "A"), _ptr(B, "B"), _rows(B, "B"),
                                _ptr(C, "C"), _rows(C, "C"), _dt(C), r_ptr, ldr, M, N, K,
                                _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                _stream(stream))
    _check(st, "gdn_gemm_bf16_ws")


def gdn_validate_metadata(query_start_loc, slot_ids, num_tokens, num_slots):
    """Host-side check of host (CPU) int32 copies of the varlen metadata."""
    qsl = query_start_loc.cpu().to(torch.int32).contiguous()
    sl = slot_ids.cpu().to(torch.int32).contiguous()
    return int(lib().gdn_validate_metadata(qsl.data_ptr(), sl.data_ptr() if sl.numel() else None,
                                           sl.numel(), int(num_tokens), int(num_slots)))


def gdn_validate_spec_metadata(query_start_loc, slot_ids, spec_slot_ids, num_tokens, num_slots):
    """Host-side check of host (CPU) int32 copies of the spec-verify metadata."""
    qsl = query_start_loc.cpu().to(torch.int32).contiguous()
    sl = slot_ids.cpu().to(torch.int32).contiguous()
    sp = spec_slot_ids.cpu().to(torch.int32).contiguous()
    return int(lib().gdn_validate_spec_metadata(
        qsl.data_ptr(), sl.data_ptr() if sl.numel() else None, sp.data_ptr() if sp.numel() else None,
        sp.shape[1] if sp.dim() == 2 else 0, sl.numel(), int(num_tokens), int(num_slots)))


def gdn_validate_snapshot_metadata(query_start_loc, slot_ids, snap_slot_ids, snap_interval,
                                   num_tokens, num_slots):
    """Host-side check of host (CPU) int32 copies of the snapshot metadata."""
    qsl = query_start_loc.cpu().to(torch.int32).contiguous()
    sl = slot_ids.cpu().to(torch.int32).contiguous()
    sp = snap_slot_ids.cpu().to(torch.int32).contiguous()
    return int(lib().gdn_validate_snapshot_metadata(
        qsl.data_ptr(), sl.data_ptr() if sl.numel() else None, sp.data_ptr() if sp.numel() else None,
        sp.shape[1] if sp.dim() == 2 else 0, int(snap_interval), sl.numel(), int(num_tokens),
        int(num_slots)))
