"""TurboQuant KV-cache vector quantization for AMD Instinct MI355X (gfx950).

The compute path is ``libtq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/tq.h``).  ``kv_cache_vector_quantize_amd.tq`` is the
thin ctypes binding over torch tensors; ``inputs`` draws seeded synthetic
workloads.  Importing the package does not load the library; the first call
into ``tq`` does, and raises if it is missing.
"""

__all__ = ["tq", "inputs"]
