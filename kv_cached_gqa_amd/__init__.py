"""KV-cached grouped-query attention for MI355X (gfx950).

The compute path is a C-ABI library of hand-written HIP kernels
(libkvc.so, declared in include/kvc.h); `kv_cached_gqa_amd.kvc` is its thin
ctypes binding. Importing the package itself loads nothing: the binding loads
the library on first import and raises if it has not been built.
"""
