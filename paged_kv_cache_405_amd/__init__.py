"""MI355X-native paged decode attention (PagedAttention) and KV append.

The compute path is a HIP library for gfx950 behind a C ABI (include/pa.h);
``paged_kv_cache_405_amd.binding`` marshals torch tensors into it.  Importing
this package loads nothing: the binding loads the library on first use and
raises if it has not been built.
"""
__all__ = ["binding", "workloads"]
