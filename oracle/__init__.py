"""CPU oracle for the Gated DeltaNet mixer core — TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 definitions of every step of the GDN mixer path, written
from the pages ("Qwen3.8-27B: from model structure to the vLLM inference
dataflow", section 01 per-layer operator table and data-structure table,
section 03 GDN state lab, section 08 evidence matrix).  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The GPU library never calls, links or loads anything here, and the
two share no code.

Parity status per function (see the oracle tests for the pins):
  conv1d_silu, l2norm, gates, gated_delta_rule, decode_step, gated_norm,
  rmsnorm, linear, residual_add, gdn_layer, spec_verify, round_bf16,
  prefill_snapshots, and (gqa.py) rope_partial, gqa_decode_paged, e4m3_decode,
  e4m3_round, e4m3_encode — pinned
  (closed forms, brute force, library reductions, worked examples printed on
  the pages).
  Absolute output values for the full-size workloads are not printed anywhere
  on the pages; beyond the pins they are parity-unpinned by construction.
"""
from .gqa import (  # noqa: F401
    e4m3_decode,
    e4m3_encode,
    e4m3_round,
    fp8_cache_round,
    gqa_decode_paged,
    rope_partial,
)
from .oracle import (  # noqa: F401
    conv1d_silu,
    conv1d_update,
    decode_step,
    gated_delta_rule,
    gated_norm,
    gates,
    gdn_layer,
    l2norm,
    linear,
    num_threads,
    prefill_snapshots,
    residual_add,
    rmsnorm,
    round_bf16,
    set_num_threads,
    silu,
    spec_verify,
    split_qkv,
)
