"""liblsa for MI355X: the LSA decode hot path (score -> select -> stage ->
attend) as hand-written HIP kernels behind the C ABI of include/lsa.h.

``learned_sparse_kv_amd.lsa`` is the ctypes binding; ``learned_sparse_kv_amd.build``
compiles ``liblsa.so`` for gfx950.  Importing the package loads nothing.
"""
__all__ = ["lsa", "build"]
