"""Thin ctypes binding of the GQA decode entry points (include/gqa.h) of libgdn.

Same rules as the GDN binding: argument marshalling only, the current torch
stream as the hipStream_t, a non-OK status raises, no fallback path.
"""
import ctypes

import numpy as np
import torch

from .gdn import GDN_BF16, GDN_FP8_E4M3, GqaDimsC, _check, _dt, _ptr, _rows, _stream, lib


def dims_c(dims) -> GqaDimsC:
    if isinstance(dims, GqaDimsC):
        return dims
    if isinstance(dims, (tuple, list)):
        return GqaDimsC(*[int(x) for x in dims])
    return GqaDimsC(int(dims.num_q_heads), int(dims.num_kv_heads), int(dims.head_dim),
                    int(dims.rotary_dim))


def gqa_decode_workspace_bytes(dims, num_reqs, max_context_len):
    d = dims_c(dims)
    return int(lib().gqa_decode_workspace_bytes(ctypes.byref(d), int(num_reqs), int(max_context_len)))


def _cache_dt(t):
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return GDN_FP8_E4M3
    raise TypeError(f"unsupported KV cache dtype {t.dtype}")


def gqa_decode_paged(dims, q, gate, k, v, k_cache, v_cache, block_tables, context_lens, page_size,
                     max_context_len, y, workspace, rope_theta=10000.0, o=None, k_scale=1.0,
                     v_scale=1.0, stream=None):
    """q, gate [R, >=Hq*D] (or [R, Hq, D]); k, v [R, >=Hkv*D] sharing one row
    stride; k_cache, v_cache [num_pages, Hkv, page_size, D], bf16 or e4m3 codes
    (uint8 / float8_e4m3fn, with k_scale, v_scale);
    block_tables int32 [R, max_pages]; context_lens int32 [R];
    y [R, Hq*D]; o optional fp32 [R, Hq, D]; workspace uint8 of
    gqa_decode_workspace_bytes bytes."""
    d = dims_c(dims)
    R = context_lens.numel()
    q2, g2 = q.reshape(R, -1) if q.is_contiguous() else q, gate.reshape(R, -1) if gate.is_contiguous() else gate
    k2, v2 = k.reshape(R, -1) if k.is_contiguous() else k, v.reshape(R, -1) if v.is_contiguous() else v
    if _rows(k2, "k") != _rows(v2, "v"):
        raise ValueError("k and v share one row stride")
    if not (q.dtype == gate.dtype == k.dtype == v.dtype):
        raise ValueError("q, gate, k and v share one dtype")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("block_tables", block_tables),
                    ("y", y), ("workspace", workspace)):
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
    if o is not None and (o.dtype != torch.float32 or not o.is_contiguous()):
        raise TypeError("o must be contiguous float32")
    cdt = _cache_dt(k_cache)
    if _cache_dt(v_cache) != cdt:
        raise TypeError("k_cache and v_cache share one dtype")
    st = lib().gqa_decode_paged(
        ctypes.byref(d), _ptr(q2, "q"), _rows(q2, "q"), _ptr(g2, "gate"), _rows(g2, "gate"),
        _ptr(k2, "k"), _ptr(v2, "v"), _rows(k2, "k"), _dt(q), _ptr(k_cache, "k_cache"),
        _ptr(v_cache, "v_cache"), cdt, float(k_scale), float(v_scale), _ptr(block_tables, "block_tables"),
        block_tables.shape[1], _ptr(context_lens, "context_lens"), R, k_cache.shape[0],
        int(page_size), int(max_context_len), float(rope_theta), _ptr(y, "y"), _dt(y),
        _ptr(o, "o"), _ptr(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "gqa_decode_paged")


def gqa_validate_decode_metadata(block_tables, context_lens, num_pages, page_size, max_context_len):
    """Host copies (CPU tensors or arrays) of the block tables and lengths;
    returns the status code (0 = OK)."""
    bt = np.ascontiguousarray(np.asarray(block_tables.cpu() if torch.is_tensor(block_tables)
                                         else block_tables, dtype=np.int32))
    ln = np.ascontiguousarray(np.asarray(context_lens.cpu() if torch.is_tensor(context_lens)
                                         else context_lens, dtype=np.int32))
    return int(lib().gqa_validate_decode_metadata(
        bt.ctypes.data, bt.shape[1], ln.ctypes.data, ln.size, int(num_pages), int(page_size),
        int(max_context_len)))
