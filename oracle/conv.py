"""Two-dimensional convolution: the CPU oracle of the library's implicit-GEMM
convolution.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.

Page "The Tensor Core" lists implicit-GEMM convolutions among the work that
reduces to a matrix product. Page "Grid 24 is not headroom" profiles a
convolution kernel next to the GEMM. Neither page writes the operation out.
The reading taken here is the convolution of deep-learning frameworks
(cross-correlation: the filter is not flipped), with zero padding, stride
and dilation:

    y[n][p][q][k] = sum_{r, s, c} x[n][p sh - ph + r dh][q sw - pw + s dw][c] w[k][r][s][c]

where x reads as zero outside its H x W extent, and P = (H + 2 ph - dh (R-1) - 1)
// sh + 1 (Q likewise). Layouts: x NHWC, w KRSC, y NPQK.

Elements are decoded to binary64 (bf16: the upper half of a binary32).
The sum runs over the filter taps (r, s) in order. Each tap contributes a
binary64 matrix product (a library primitive) over the C channels. W is
sum |x w| over the same terms and scales the parity tolerance.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def out_size(H: int, W: int, R: int, S: int, ph: int, pw: int, sh: int, sw: int, dh: int,
             dw: int) -> Tuple[int, int]:
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    return P, Q


def decode_bf16(codes: np.ndarray) -> np.ndarray:
    """uint16 bf16 codes -> binary64."""
    c = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << 16
    return c.view(np.float32).astype(np.float64)


def _padded(x: np.ndarray, ph: int, pw: int) -> np.ndarray:
    N, H, W, C = x.shape
    xp = np.zeros((N, H + 2 * ph, W + 2 * pw, C))
    xp[:, ph:ph + H, pw:pw + W, :] = x
    return xp


def _window(xp: np.ndarray, r: int, s: int, P: int, Q: int, sh: int, sw: int, dh: int,
            dw: int) -> np.ndarray:
    """The input pixels tap (r, s) meets for every output pixel:
    xp[n][p sh + r dh][q sw + s dw][c], an N x P x Q x C array."""
    h0, w0 = r * dh, s * dw
    return xp[:, h0:h0 + sh * (P - 1) + 1:sh, w0:w0 + sw * (Q - 1) + 1:sw, :]


def conv2d(x: np.ndarray, w: np.ndarray, ph: int = 0, pw: int = 0, sh: int = 1, sw: int = 1,
           dh: int = 1, dw: int = 1, alpha: float = 1.0):
    """x: N x H x W x C values (binary64 or bf16 codes as uint16), w: K x R x
    S x C likewise.  Returns (y, W) as binary64 N x P x Q x K arrays."""
    xv = decode_bf16(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    wv = decode_bf16(w) if np.asarray(w).dtype == np.uint16 else np.asarray(w, dtype=np.float64)
    N, H, W_, C = xv.shape
    K, R, S, C2 = wv.shape
    if C2 != C:
        raise ValueError("channel counts differ")
    P, Q = out_size(H, W_, R, S, ph, pw, sh, sw, dh, dw)
    if P < 1 or Q < 1:
        raise ValueError("empty output")
    xp = _padded(xv, ph, pw)
    y = np.zeros((N, P, Q, K))
    mag = np.zeros((N, P, Q, K))
    for r in range(R):
        for s in range(S):
            win = _window(xp, r, s, P, Q, sh, sw, dh, dw).reshape(-1, C)
            tap = wv[:, r, s, :]
            y += (win @ tap.T).reshape(N, P, Q, K)
            mag += (np.abs(win) @ np.abs(tap).T).reshape(N, P, Q, K)
    return alpha * y, abs(alpha) * mag


def conv2d_entries(x: np.ndarray, w: np.ndarray, idx: np.ndarray, ph: int = 0, pw: int = 0,
                   sh: int = 1, sw: int = 1, dh: int = 1, dw: int = 1):
    """Selected outputs idx[t] = (n, p, q, k), each its own R x S x C sum."""
    xv = decode_bf16(x) if np.asarray(x).dtype == np.uint16 else np.asarray(x, dtype=np.float64)
    wv = decode_bf16(w) if np.asarray(w).dtype == np.uint16 else np.asarray(w, dtype=np.float64)
    N, H, W_, C = xv.shape
    K, R, S, _ = wv.shape
    out = np.zeros(len(idx))
    mag = np.zeros(len(idx))
    for t, (n, p, q, k) in enumerate(np.asarray(idx, dtype=np.int64)):
        acc = 0.0
        am = 0.0
        for r in range(R):
            h = p * sh - ph + r * dh
            if h < 0 or h >= H:
                continue
            for s in range(S):
                ww = q * sw - pw + s * dw
                if ww < 0 or ww >= W_:
                    continue
                prod = xv[n, h, ww, :] * wv[k, r, s, :]
                acc += prod.sum()
                am += np.abs(prod).sum()
        out[t] = acc
        mag[t] = am
    return out, mag
