"""Paged KV-cache decode path for MI355X (gfx950).

The HIP kernels live in ``csrc/`` and are exported through the C-ABI library
``libpa.so`` (declared in ``include/pa.h``).  :mod:`paged_kv_cache_414_amd.ops`
holds the thin Python binding; nothing is loaded until it is imported.
"""

__all__ = ["ops", "blocks", "workloads", "metrics"]
