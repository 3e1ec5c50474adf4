"""Block-scaled ("microscaled") 8-bit products: the CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.

Page "The Tensor Core", the low-precision input table, lists microscaled
formats as the row after the Hopper FP8 pair. The pages stop at the name.
The reading taken here is the OCP Microscaling Formats (MX) specification,
version 1.0:

* a block is 32 consecutive elements along the contraction dimension K,
  all sharing one scale;
* the scale is an E8M0 code e, whose value is 2^(e - 127); e = 255 is NaN;
* the elements are E4M3 or E5M2 codes, decoded as in ``gemm_oracle.c``, or
  FP4 E2M1 codes (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
  exponent field 0 is subnormal, m * 0.5; no infinity or NaN), two per byte
  with element 2i in the low nibble of byte i, or FP6 E2M3 codes (2
  exponent bits with bias 1, 3 mantissa bits) or E3M2 codes (3 exponent bits
  with bias 3, 2 mantissa bits), no infinity or NaN, packed as a
  little-endian bit stream (element i in bits 6i .. 6i+5 of its row);
* an element's value is scale * element.

For A (M x K) each row has ceil(K/32) scales. For B (K x N) each column has
ceil(K/32) scales. The product is written out directly:

    C[i][j] = alpha * sum_k (2^(sa[i][k/32] - 127) a(i,k)) (2^(sb[j][k/32] - 127) b(k,j))
    W[i][j] = |alpha| * sum_k |same term|

Element values come from the C oracle's decoders, which are pinned
exhaustively against torch's casts. Each scaled element is then exact in
binary64: a power of two times a short significand, far inside binary64's
range. The K-term sum is a binary64 matrix product (a library primitive), so
the only rounding is binary64 summation.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import reference

BLOCK = 32


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes -> binary64: 2^(e - 127), NaN for e = 255."""
    e = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (low nibble) -> binary64."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(sign == 1, -mag, mag)


def _decode_minifloat(codes: np.ndarray, ebits: int, mbits: int, bias: int) -> np.ndarray:
    """Sign, ebits exponent bits, mbits mantissa bits; exponent field 0 is
    subnormal; every other code is a normal number (no infinity or NaN)."""
    width = 1 + ebits + mbits
    c = np.asarray(codes, dtype=np.int64) & ((1 << width) - 1)
    sign = c >> (width - 1)
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = c & ((1 << mbits) - 1)
    frac = m / float(1 << mbits)
    mag = np.where(e == 0, np.ldexp(frac, 1 - bias), np.ldexp(1.0 + frac, e - bias))
    return np.where(sign == 1, -mag, mag)


def decode_e2m3(codes: np.ndarray) -> np.ndarray:
    """6-bit E2M3 codes -> binary64."""
    return _decode_minifloat(codes, 2, 3, 1)


def decode_e3m2(codes: np.ndarray) -> np.ndarray:
    """6-bit E3M2 codes -> binary64."""
    return _decode_minifloat(codes, 3, 2, 3)


def unpack_fp6(packed: np.ndarray) -> np.ndarray:
    """rows x 3K/4 bytes -> rows x K 6-bit codes (little-endian bit stream:
    element i in bits 6i .. 6i+5)."""
    b = np.asarray(packed, dtype=np.uint8)
    rows, nbytes = b.shape
    bits = np.unpackbits(b, axis=1, bitorder="little")          # bit j of the row
    k = nbytes * 8 // 6
    bits = bits[:, :k * 6].reshape(rows, k, 6).astype(np.int64)
    return (bits * (1 << np.arange(6))).sum(axis=2).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """rows x K/2 bytes -> rows x K codes (element 2i = low nibble)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def _element_table(fmt: str) -> np.ndarray:
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    if fmt == "e2m1":
        return decode_e2m1(codes)
    if fmt == "e2m3":
        return decode_e2m3(codes)
    if fmt == "e3m2":
        return decode_e3m2(codes)
    if fmt == "e4m3":
        return reference.decode_e4m3(codes)
    if fmt == "e5m2":
        return reference.decode_e5m2(codes)
    raise ValueError("block-scaled element format must be e4m3, e5m2, e2m3, e3m2 or e2m1, not %r" % (fmt,))


def scaled_operand(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """Rows x K element codes (rows x K/2 packed bytes for e2m1, rows x
    3K/4 for e2m3 / e3m2) and
    rows x ceil(K/32) E8M0 scales -> the binary64 values
    2^(s - 127) * element, rows x K."""
    codes = np.asarray(codes, dtype=np.uint8)
    if fmt == "e2m1":
        codes = unpack_fp4(codes)
    elif fmt in ("e2m3", "e3m2"):
        codes = unpack_fp6(codes)
    rows, K = codes.shape
    nb = -(-K // BLOCK)
    scales = np.asarray(scales, dtype=np.uint8)
    if scales.shape != (rows, nb):
        raise ValueError("scales must be rows x ceil(K/32) = %s, got %s" % ((rows, nb), scales.shape))
    vals = _element_table(fmt)[codes]
    per_k = np.repeat(decode_e8m0(scales), BLOCK, axis=1)[:, :K]
    return vals * per_k


def gemm(A: np.ndarray, sa: np.ndarray, B: np.ndarray, sb: np.ndarray, fmt_a: str = "e4m3",
         fmt_b: Optional[str] = None, alpha: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """A: M x K codes (row-major; M x K/2 bytes for e2m1), sa: M x ceil(K/32);
    B: N x K codes (column j of B is row j), sb: N x ceil(K/32). Returns
    (C, W), both binary64 M x N."""
    fmt_b = fmt_a if fmt_b is None else fmt_b
    a = scaled_operand(A, sa, fmt_a)
    b = scaled_operand(B, sb, fmt_b)
    C = alpha * (a @ b.T)
    W = abs(alpha) * (np.abs(a) @ np.abs(b).T)
    return C, W


def gemm_entries(A: np.ndarray, sa: np.ndarray, B: np.ndarray, sb: np.ndarray, rows: np.ndarray,
                 cols: np.ndarray, fmt_a: str = "e4m3", fmt_b: Optional[str] = None,
                 alpha: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Selected entries (rows[t], cols[t]) of the same product, each its own
    K-term dot product."""
    fmt_b = fmt_a if fmt_b is None else fmt_b
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    a = scaled_operand(np.asarray(A)[rows], np.asarray(sa)[rows], fmt_a)
    b = scaled_operand(np.asarray(B)[cols], np.asarray(sb)[cols], fmt_b)
    c = alpha * np.einsum("tk,tk->t", a, b)
    w = abs(alpha) * np.einsum("tk,tk->t", np.abs(a), np.abs(b))
    return c, w
