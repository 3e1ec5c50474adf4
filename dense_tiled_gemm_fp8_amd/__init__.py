"""dense_tiled_gemm_fp8_amd: the libgemm355 tiled GEMM for MI355X (gfx950).

The compute path lives in the HIP shared library ``libgemm355.so`` built from
``csrc/``; :mod:`dense_tiled_gemm_fp8_amd.gemm355` is a thin ctypes binding to
its C ABI.  Importing this package loads nothing; importing ``gemm355`` loads
the library and fails loudly if it has not been built.
"""
__all__ = ["gemm355", "inputs", "build"]
