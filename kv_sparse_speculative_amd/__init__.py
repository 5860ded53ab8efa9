"""MI355X-native hot path of sparse-KV self-speculative decoding.

The compute lives in a C-ABI shared library of hand-written HIP kernels for gfx950
(``libkvss.so``); ``kv_sparse_speculative_amd.kvss`` is its thin Python binding. Importing
this package does not load the library; the binding loads it on first use and raises if it
is missing.
"""
