"""Paged KV-cache hot path for AMD Instinct MI355X (gfx950).

``paged_kv_cache_378_amd._lib`` is the ctypes binding of libpa.so (the C ABI in
include/pa.h): host block manager, cache write, copy-on-write block copy,
split-K paged decode and chunked-query paged attention.  ``workloads`` holds the
seeded synthetic input generators.  ``build`` compiles libpa.so in-tree.

The binding is imported lazily (``from paged_kv_cache_378_amd import _lib``) so
that the generators can be used where the library is not built; the binding
itself refuses to import without libpa.so.
"""

__all__ = ["build", "workloads"]
