"""MI355X-native Gated DeltaNet mixer core.

The compute lives in ``libgdn.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/gdn.h``); ``hybrid_linear_attention_amd.gdn`` is the thin
ctypes binding that marshals torch tensors into those calls.  Importing the
package does not load the library; the binding raises if it is missing.
"""
__all__ = ["gdn", "workloads"]
