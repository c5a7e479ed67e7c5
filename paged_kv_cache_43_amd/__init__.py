"""Decode-step paged attention for MI355X (gfx950).

``paged_kv_cache_43_amd.pf`` is the Python binding of the C-ABI library
``libpf.so`` (same function names as ``include/pf.h``); importing it fails
loudly if the library has not been built.  ``paged_kv_cache_43_amd.inputs``
draws the seeded synthetic workloads.
"""
