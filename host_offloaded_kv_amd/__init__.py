"""MI355X-native HiSparse decode path: RESOLVE against a B-slot device hot
buffer with LRU replacement and zero-copy miss fetches from a pinned host KV
pool, then sparse MLA decode attention over the resolved rows.

The compute lives in the HIP library ``libhisparse.so`` (C ABI in
``include/hisparse.h``); ``hisparse`` is its ctypes binding.
"""
