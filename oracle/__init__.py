"""CPU oracle for the tiled dense matrix product.

TEST INFRASTRUCTURE ONLY.  The product library never imports, calls, links or
executes anything in this package.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code with the GPU path
and does not import the product package.

Two parts:

* ``gemm_oracle.c`` (wrapped by :mod:`oracle.reference`): the plain binary64
  triple-loop product C = alpha * A @ B, plus the magnitude W = |alpha| *
  sum_k |a_ik b_kj|.  It decodes bf16 and E4M3 from their bit definitions.
* :mod:`oracle.bookkeeping`: exact-rational tile bookkeeping: the FLOP count,
  the tile grid G, wave efficiency, padding efficiency, K-slices, resident
  workgroups and schedule efficiency.

Page citations are given as the page title plus the section or equation.
"""
