"""Quantized KV cache with fused decode attention for AMD Instinct MI355X (gfx950).

The compute path is libkvq.so (hand-written HIP kernels behind the C ABI in include/kvq.h);
``quantized_kv_cache_07_amd.kvq`` is its thin ctypes binding.  Import that module to use it: it
raises ImportError when the library has not been built.
"""
