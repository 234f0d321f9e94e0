"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute lives in ``libpagedkv.so`` (hand-written HIP kernels behind a C ABI, declared
in ``include/pagedkv.h``); ``paged_kv_cache_376_amd.binding`` marshals torch tensors into
it.  ``workloads`` draws the seeded synthetic inputs.  Importing the package loads nothing
native; the library is opened on first use of the binding.
"""

__all__ = ["binding", "workloads"]
