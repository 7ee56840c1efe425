"""ART decode attention over a paged KV cache, MI355X (gfx950) native.

The compute path is the C-ABI shared library built from ``csrc/`` (hand-written
HIP kernels for gfx950); ``kv_cache_run_amd.art`` is its thin ctypes binding.
Nothing is imported eagerly so that the input generator can be used on
machines without a GPU.
"""
