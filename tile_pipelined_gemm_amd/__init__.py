"""tile_pipelined_gemm_amd: persistent role-specialised fused GEMM kernels for MI355X.

The compute path is libmk.so (hand-written HIP for gfx950) behind a C ABI
declared in include/mk.h; ``tile_pipelined_gemm_amd.mk`` is a thin ctypes
binding with the same entry-point names.  Importing this package does not load
the library; ``mk.load()`` does and fails loudly if it is missing.
"""
__all__ = ["mk", "build"]
