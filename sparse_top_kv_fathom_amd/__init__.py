"""MI355X (gfx950) Fathom key scan: encode, plan, scan and top-k behind a C ABI.

The calls follow "Fathom: Per-Query Read Depth for Sparse Decoding over
Offloaded KV Caches" (§3.2 bit-plane K store, §3.3 per-query read depth,
§2 per-head top-k, §3.5 the KLT-rotated store, §3.6 the host-resident
store).  The work runs in hand-written HIP kernels in
libfathom.so (include/fathom.h); this package is a thin ctypes binding that
takes torch device tensors.  Importing a call loads the library and raises if
it has not been built.
"""
_EXPORTS = ("encode", "plan", "append_plan", "plan_fixed", "PLAN_MODES", "scan", "scan_topk", "scan_topk_workspace", "gather", "klt_fit", "klt_fit_workspace",
            "klt_rotate_keys", "klt_rotate_queries", "topk", "topk_noalloc", "topk_workspace_bytes", "topk_workspace",
            "test_cut_hooks",
            "empty_store", "store_shapes", "FathomError", "lib", "STATUS", "EXPORTED")

__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
