"""Jensen-bias-corrected INT2/INT4 KV-cache attention for AMD MI355X (gfx950).

The compute lives in ``libkvq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/kvq.h``).  ``bit_kv_cache_03_amd.kvq`` is the thin
ctypes binding; importing it loads the library and fails loudly when it has
not been built.  ``bit_kv_cache_03_amd.workloads`` draws the seeded synthetic
inputs.
"""
__all__ = ["kvq", "workloads"]
