"""MI355X-native paged KV-cache decode attention (PagedAttention decode).

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, built to ``libpa.so``), declared in ``include/pa.h``.
``paged_kv_cache_163_amd.pa`` is a thin ctypes binding over it (argument
marshalling only).  ``paged_kv_cache_163_amd.workloads`` builds the seeded
synthetic decode batches used by the tests and the benchmark.

Importing this package loads nothing; importing ``.pa`` loads ``libpa.so`` and
raises if it has not been built.
"""
