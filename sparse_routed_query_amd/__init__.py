"""GQE (Grouped Query Experts) attention forward for AMD MI355X (gfx950).

The compute lives in ``libgqe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/gqe.h``); ``sparse_routed_query_amd.gqe`` is its thin
Python binding.
"""
