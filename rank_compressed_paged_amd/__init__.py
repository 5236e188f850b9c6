"""MI355X (gfx950) attention over a paged, low-rank-compressed KV cache.

The compute path lives in the HIP library ``libstarkv.so`` behind the C ABI
declared in ``include/starkv.h``; ``rank_compressed_paged_amd.starkv`` is the
thin Python binding over it.  Importing the package itself loads nothing, so
the seeded workload generators can be used on machines without the library.
"""
__all__ = ["workloads", "metrics"]
