"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The GPU operations live in :mod:`paged_kv_cache_298_amd.pa`, a thin ctypes binding over
the C-ABI library ``libpa.so`` built from ``csrc/``; importing that module fails loudly if
the library is missing. :mod:`paged_kv_cache_298_amd.workloads` only draws seeded inputs.
"""
__all__ = ["pa", "workloads"]
