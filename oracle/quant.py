"""Per-tensor quantisation to 8-bit floats (E4M3FN, E5M2): the CPU oracle of
the library's quantiser.

TEST INFRASTRUCTURE ONLY: imported by the tests and the benchmark's
CPU-baseline leg, never by the product library.

What it computes (the FP8 pair of the Hopper row of the input/accumulate
table on page "The Tensor Core"; page "10. Tensor Cores, shapes, and tile
alignment", section "Practical shape sweep", on judging a GEMM with its
quantisation included), for one tensor x of binary32 values:

    amax = max |x|
    s    = amax / F   in binary32 (s = 1 if amax == 0), F = 448 or 57344
    t    = x / s      in binary32, then clamped to [-F, F]
    q    = the code whose value is nearest to t; on a tie, the code with the
           even mantissa (lowest bit 0); the code's sign is t's sign bit

The nearest code is found by searching the table of every finite
non-negative value of the format, decoded by the C oracle's decoders (which
are pinned exhaustively against torch's casts); nothing here rounds bits.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import reference

FMAX = {"e4m3": 448.0, "e5m2": 57344.0}


def _table(fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """Codes 0x00..0x7F that are finite, and their values (ascending)."""
    codes = np.arange(128, dtype=np.uint16).astype(np.uint8)
    dec = reference.decode_e4m3(codes) if fmt == "e4m3" else reference.decode_e5m2(codes)
    keep = np.isfinite(dec)
    vals, cs = dec[keep], codes[keep]
    order = np.argsort(vals, kind="stable")
    return vals[order], cs[order]


def encode(t: np.ndarray, fmt: str) -> np.ndarray:
    """Nearest code to each binary32 value t (|t| <= F), ties to the even
    code, sign from t's sign bit."""
    t = np.asarray(t, dtype=np.float32)
    vals, cs = _table(fmt)
    a = np.abs(t.astype(np.float64)).reshape(-1)
    if np.any(a > FMAX[fmt]):
        raise ValueError("value beyond the format's largest finite magnitude")
    hi = np.searchsorted(vals, a, side="left")           # vals[hi-1] < a <= vals[hi]
    hi = np.clip(hi, 1, len(vals) - 1)
    lo = hi - 1
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = dhi < dlo
    tie = dhi == dlo
    # on a tie, the even code of the two (codes of neighbouring values differ by 1)
    pick_hi = np.where(tie, (cs[hi] & 1) == 0, pick_hi)
    mag = np.where(pick_hi, cs[hi], cs[lo]).astype(np.uint8)
    sign = np.signbit(t.reshape(-1)).astype(np.uint8) << 7
    return (mag | sign).reshape(t.shape)


def quantize(x: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.float32]:
    """(codes, s) of one tensor, following the definition above."""
    x32 = np.asarray(x, dtype=np.float32)
    F = np.float32(FMAX[fmt])
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    s = np.float32(amax / F) if amax > 0 else np.float32(1.0)
    t = np.clip(np.float32(x32 / s), -F, F).astype(np.float32)
    return encode(t, fmt), s


def quantize_batch(x: np.ndarray, n: int, batch: int, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """Tensors x[g*n : (g+1)*n] for g < batch; returns (codes, scales)."""
    x32 = np.asarray(x, dtype=np.float32).reshape(-1)
    q = np.zeros(n * batch, dtype=np.uint8)
    s = np.zeros(batch, dtype=np.float32)
    for g in range(batch):
        q[g * n:(g + 1) * n], s[g] = quantize(x32[g * n:(g + 1) * n], fmt)
    return q, s
