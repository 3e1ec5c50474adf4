"""CPU oracle for the tiled dense matrix product.

TEST INFRASTRUCTURE ONLY.  The product library never imports, calls, links or
executes anything in this package.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code with the GPU path
and does not import the product package.

Five parts:

* ``gemm_oracle.c`` (wrapped by :mod:`oracle.reference`): the plain binary64
  triple-loop product C = alpha * A @ B, plus the magnitude W = |alpha| *
  sum_k |a_ik b_kj|.  It decodes bf16, E4M3 and E5M2 from their bit
  definitions (A and B may use different 8-bit formats).
* :mod:`oracle.quant`: per-tensor quantisation to E4M3 / E5M2 (amax, scale,
  nearest code with ties to even) by search over the decoded code table.
* :mod:`oracle.mx`: the block-scaled (microscaled) 8-bit product: 32-element
  blocks along K sharing one E8M0 power-of-two scale, written out as the
  scaled elements' binary64 dot products.
* :mod:`oracle.conv`: two-dimensional convolution (NHWC images, KRSC
  filters, padding, stride, dilation) as tap-by-tap binary64 products.
* :mod:`oracle.bookkeeping`: exact-rational tile bookkeeping: the FLOP count,
  the tile grid G, wave efficiency, padding efficiency, K-slices, resident
  workgroups and schedule efficiency.

Page citations are given as the page title plus the section or equation.
"""
