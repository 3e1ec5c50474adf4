"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.

This module holds no part of the product's arithmetic: it draws random numbers
with numpy's PCG64 and rounds them to the element formats with torch's CPU
casts (round-to-nearest-even).  The GPU path and the CPU oracle both consume
the raw codes it returns.

Seeds: ``1000*workload + 10*shape_index + {0: A, 1: B}``.

Storage convention (the layouts of the sweep command in section "Practical
shape sweep" of page "10. Tensor Cores, shapes, and tile alignment": A
row-major, B column-major):
  * A is M x K row-major, lda = K  (array shape (M, K))
  * B is K x N column-major, ldb = K (array shape (N, K): column j of B is
    row j of the array)
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

E4M3_MAX = 448.0
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}
_TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def seed_for(workload: int, shape_index: int, operand: int) -> int:
    return 1000 * workload + 10 * shape_index + operand


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def draw(gen: np.random.Generator, shape, dist: str, K: Optional[int] = None) -> np.ndarray:
    """binary64 samples: 'uniform' U[-1,1], 'normal' N(0,1), 'normal_sqrtk'
    N(0,1)/sqrt(K)."""
    if dist == "uniform":
        return gen.uniform(-1.0, 1.0, size=shape)
    if dist == "normal":
        return gen.standard_normal(size=shape)
    if dist == "normal_sqrtk":
        if not K:
            raise ValueError("normal_sqrtk needs K")
        return gen.standard_normal(size=shape) / np.sqrt(K)
    raise ValueError("unknown distribution %r" % dist)


def to_bf16_codes(x: np.ndarray) -> np.ndarray:
    """binary64 -> binary32 (RNE) -> bf16 (RNE); returns uint16 codes."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_fp8_codes(x: np.ndarray, fmt: str, scale: Optional[float] = None) -> Tuple[np.ndarray, float]:
    """Per-tensor quantisation to OCP E4M3FN or E5M2 (the input recipe).  In
    binary32: s = amax|x|/F (unless given; F = 448 or 57344),
    q = rne(clamp(x/s, -F, F)) by torch's CPU cast.  Returns (uint8 codes,
    s); x is approximately s * decode(q)."""
    F = FP8_MAX[fmt]
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if scale is None:
        amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
        scale = float(np.float32(amax) / np.float32(F)) if amax > 0 else 1.0
    s32 = np.float32(scale)
    y = np.clip(x32 / s32, -F, F).astype(np.float32)
    q = torch.from_numpy(y).to(_TORCH_FP8[fmt]).view(torch.uint8).numpy()
    return q, float(s32)


def to_e4m3_codes(x: np.ndarray, scale: Optional[float] = None) -> Tuple[np.ndarray, float]:
    """to_fp8_codes for E4M3FN."""
    return to_fp8_codes(x, "e4m3", scale)


FP8_EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2, "e2m3": 2, "e3m2": 4}   # exponent of the largest finite value
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # codes 0..7 (OCP FP4)


def to_e2m1_codes(y: np.ndarray) -> np.ndarray:
    """Round to the nearest E2M1 value, ties to the even code, saturating
    at 6; returns 4-bit codes (sign in bit 3) as uint8.  The value steps are
    0.5 below 2, 1 in [2, 4) and 2 in [4, 6], and an even code is an even
    multiple of the step, so rint (ties to even) on the scaled magnitude
    picks it."""
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), 6.0)
    q = np.where(mag < 2.0, np.rint(mag * 2.0) / 2.0,
                 np.where(mag < 4.0, np.rint(mag), np.minimum(2.0 * np.rint(mag / 2.0), 6.0)))
    code = np.searchsorted(E2M1_VALUES, q).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 3)


def _fp6_grid(fmt: str) -> np.ndarray:
    """Non-negative values of the 6-bit format, indexed by code 0..31."""
    eb, mb, bias = (2, 3, 1) if fmt == "e2m3" else (3, 2, 3)
    vals = []
    for code in range(32):
        e, m = code >> mb, code & ((1 << mb) - 1)
        vals.append(m / 2.0 ** mb * 2.0 ** (1 - bias) if e == 0 else (1 + m / 2.0 ** mb) * 2.0 ** (e - bias))
    return np.array(vals)


def to_fp6_codes(y: np.ndarray, fmt: str) -> np.ndarray:
    """Round to the nearest E2M3 / E3M2 value, ties to the even code,
    saturating at the largest; 6-bit codes (sign in bit 5) as uint8."""
    grid = _fp6_grid(fmt)
    y = np.asarray(y, dtype=np.float64)
    mag = np.minimum(np.abs(y), grid[-1])
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 1, 31)
    lo = hi - 1
    dlo, dhi = mag - grid[lo], grid[hi] - mag
    pick = np.where(dhi == dlo, (hi & 1) == 0, dhi < dlo)
    code = np.where(pick, hi, lo).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 5)


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """rows x K 6-bit codes -> rows x 3K/4 bytes, a little-endian bit
    stream (element i in bits 6i .. 6i+5)."""
    c = np.asarray(codes, dtype=np.uint8)
    rows, K = c.shape
    bits = ((c[:, :, None] >> np.arange(6)) & 1).astype(np.uint8).reshape(rows, K * 6)
    return np.packbits(bits, axis=1, bitorder="little")


def to_mx_fp6_codes(x: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """Block-scaled FP6 quantisation (OCP MX v1.0 conversion, as
    to_mx_codes with emax 2 for E2M3 and 4 for E3M2): (rows x 3K/4 packed
    bytes, rows x K/32 scale codes)."""
    x64 = np.asarray(x, dtype=np.float64)
    rows, K = x64.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = x64.reshape(rows, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, e = np.frexp(amax)
    code = np.where(amax > 0, e - 1 - FP8_EMAX[fmt] + 127, 127)
    code = np.clip(code, 0, 254).astype(np.uint8)
    scale = np.ldexp(1.0, code.astype(np.int64) - 127)
    q = to_fp6_codes((blocks / scale[:, :, None]).reshape(rows, K), fmt)
    return pack_fp6(q), code


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """rows x K 4-bit codes -> rows x K/2 bytes, element 2i in the low
    nibble of byte i."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def to_mx_fp4_codes(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Block-scaled FP4 quantisation (OCP MX v1.0 conversion, as
    to_mx_codes with emax 2): returns (rows x K/2 packed bytes, rows x K/32
    scale codes)."""
    x64 = np.asarray(x, dtype=np.float64)
    rows, K = x64.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = x64.reshape(rows, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, e = np.frexp(amax)
    code = np.where(amax > 0, e - 1 - FP8_EMAX["e2m1"] + 127, 127)
    code = np.clip(code, 0, 254).astype(np.uint8)
    scale = np.ldexp(1.0, code.astype(np.int64) - 127)
    q = to_e2m1_codes((blocks / scale[:, :, None]).reshape(rows, K))
    return pack_nibbles(q), code


def to_mx_codes(x: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """Block-scaled quantisation of a rows x K array (the input recipe of
    the block-scaled dtypes; OCP MX v1.0 conversion): for each block of 32
    values along K, the E8M0 scale is 2^(floor(log2 amax) - emax) with emax
    the element format's largest exponent (8 for E4M3, 15 for E5M2), code
    floor(log2 amax) - emax + 127 clamped to [0, 254] (127 for an all-zero
    block); the elements are x / scale clamped to the format's largest
    magnitude and rounded to nearest even by torch's CPU cast.  K must be a
    multiple of 32.  Returns (uint8 element codes rows x K, uint8 scale
    codes rows x K / 32)."""
    x64 = np.asarray(x, dtype=np.float64)
    rows, K = x64.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = x64.reshape(rows, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, e = np.frexp(amax)                 # amax = m 2^e, 0.5 <= m < 1
    code = np.where(amax > 0, e - 1 - FP8_EMAX[fmt] + 127, 127)
    code = np.clip(code, 0, 254).astype(np.uint8)
    scale = np.ldexp(1.0, code.astype(np.int64) - 127)
    F = FP8_MAX[fmt]
    y = np.clip(blocks / scale[:, :, None], -F, F).reshape(rows, K).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(y)).to(_TORCH_FP8[fmt]).view(torch.uint8).numpy()
    return q, code


def small_int_codes(gen: np.random.Generator, shape, fmt: str, lo: int = -4,
                    hi: int = 4) -> np.ndarray:
    """Integers in [lo, hi], exactly representable in bf16, E4M3 and E5M2
    (fmt "e5m2" gives E5M2 codes, any other 8-bit name E4M3 codes)."""
    v = gen.integers(lo, hi + 1, size=shape).astype(np.float64)
    if fmt == "bf16":
        return to_bf16_codes(v)
    if fmt == "e2m1":
        # integers of E2M1: 0, 1, 2, 3, 4, 6 (packed two per byte)
        v = np.where(np.abs(v) == 5, np.sign(v) * 4, v)
        return pack_nibbles(to_e2m1_codes(v))
    if fmt in ("e2m3", "e3m2"):
        # every integer up to 7 is an E2M3 value and up to 8 an E3M2 value
        return pack_fp6(to_fp6_codes(v, fmt))
    q, _ = to_fp8_codes(v, "e5m2" if fmt == "e5m2" else "e4m3", scale=1.0)
    return q


def codes_to_torch(codes: np.ndarray, fmt: Optional[str] = None) -> torch.Tensor:
    """View raw codes as a torch tensor of the matching element type (uint8
    codes are E4M3 unless fmt is "e5m2")."""
    if codes.dtype == np.uint16:
        return torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16)
    if codes.dtype == np.uint8:
        return torch.from_numpy(codes).view(_TORCH_FP8["e5m2" if fmt == "e5m2" else "e4m3"])
    raise TypeError("codes must be uint16 (bf16) or uint8 (E4M3 / E5M2)")


def sha256(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


@dataclass
class Operands:
    """One GEMM's operands as raw codes in the storage convention above."""
    M: int
    N: int
    K: int
    fmt: str                      # "bf16", "e4m3", "e5m2" or "e4m3e5m2" (A E4M3, B E5M2);
                                  # "mx" + one of the 8-bit names, "mxfp4",
                                  # "mxfp6e2m3" or "mxfp6e3m2": block-scaled
                                  # (FP4 rows hold K/2 bytes, FP6 rows 3K/4)
    A: np.ndarray                 # (batch, M, K) or (M, K)
    B: np.ndarray                 # (batch, N, K) or (N, K)  (column-major B)
    scale_a: List[float] = field(default_factory=list)
    scale_b: List[float] = field(default_factory=list)
    seeds: Tuple[int, int] = (0, 0)
    # block-scaled formats: E8M0 scale codes, (batch,) M x K/32 and N x K/32
    bsa: Optional[np.ndarray] = None
    bsb: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return self.A.shape[0] if self.A.ndim == 3 else 1

    @property
    def mx(self) -> bool:
        return self.fmt.startswith("mx")

    @property
    def elem(self) -> str:
        """The element format name without the block-scaling prefix."""
        return self.fmt[2:] if self.mx else self.fmt

    @property
    def fmt_a(self) -> str:
        if self.elem.startswith("fp6"):
            return self.elem[3:]
        if self.elem == "fp4":
            return "e2m1"
        return "e4m3" if self.elem == "e4m3e5m2" else self.elem

    @property
    def fmt_b(self) -> str:
        if self.elem.startswith("fp6"):
            return self.elem[3:]
        if self.elem == "fp4":
            return "e2m1"
        return "e5m2" if self.elem == "e4m3e5m2" else self.elem


def make_operands(M: int, N: int, K: int, fmt: str, dist: str, seed_a: int,
                  seed_b: int, batch: int = 0) -> Operands:
    """Draw A (M x K) and B (K x N, column-major) with separate seeds; for a
    batch, entry g of each is drawn in turn from the same generator."""
    ga, gb = rng(seed_a), rng(seed_b)
    nb = max(batch, 1)
    As, Bs, sa, sb = [], [], [], []
    bsa_l, bsb_l = [], []
    for _ in range(nb):
        xa = draw(ga, (M, K), dist, K)
        xb = draw(gb, (N, K), dist, K)
        if fmt == "bf16":
            As.append(to_bf16_codes(xa))
            Bs.append(to_bf16_codes(xb))
            sa.append(1.0)
            sb.append(1.0)
        elif fmt in ("mxfp6e2m3", "mxfp6e3m2"):
            f6 = fmt[5:]
            qa, ca = to_mx_fp6_codes(xa, f6)
            qb, cb = to_mx_fp6_codes(xb, f6)
            As.append(qa)
            Bs.append(qb)
            sa.append(1.0)
            sb.append(1.0)
            bsa_l.append(ca)
            bsb_l.append(cb)
        elif fmt == "mxfp4":
            qa, ca = to_mx_fp4_codes(xa)
            qb, cb = to_mx_fp4_codes(xb)
            As.append(qa)
            Bs.append(qb)
            sa.append(1.0)
            sb.append(1.0)
            bsa_l.append(ca)
            bsb_l.append(cb)
        elif fmt.startswith("mx"):
            fa = "e5m2" if fmt == "mxe5m2" else "e4m3"
            fb = "e4m3" if fmt == "mxe4m3" else "e5m2"
            qa, ca = to_mx_codes(xa, fa)
            qb, cb = to_mx_codes(xb, fb)
            As.append(qa)
            Bs.append(qb)
            sa.append(1.0)
            sb.append(1.0)
            bsa_l.append(ca)
            bsb_l.append(cb)
        elif fmt in ("e4m3", "e5m2", "e4m3e5m2"):
            qa, s_a = to_fp8_codes(xa, "e4m3" if fmt != "e5m2" else "e5m2")
            qb, s_b = to_fp8_codes(xb, "e5m2" if fmt != "e4m3" else "e4m3")
            As.append(qa)
            Bs.append(qb)
            sa.append(s_a)
            sb.append(s_b)
        else:
            raise ValueError(fmt)
    if batch:
        A, B = np.stack(As), np.stack(Bs)
        bsa = np.stack(bsa_l) if bsa_l else None
        bsb = np.stack(bsb_l) if bsb_l else None
    else:
        A, B = As[0], Bs[0]
        bsa = bsa_l[0] if bsa_l else None
        bsb = bsb_l[0] if bsb_l else None
    return Operands(M, N, K, fmt, A, B, sa, sb, (seed_a, seed_b), bsa, bsb)


def conv_operands(N: int, H: int, W: int, C: int, K: int, R: int, S: int, dist: str, seed_x: int,
                  seed_w: int) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 codes of NHWC images x and KRSC filters w ('normal_sqrtk' scales
    by the R S C terms of each output)."""
    x = draw(rng(seed_x), (N, H, W, C), dist, R * S * C)
    w = draw(rng(seed_w), (K, R, S, C), dist, R * S * C)
    return to_bf16_codes(x), to_bf16_codes(w)


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload: shapes, element format, value recipe."""
    index: int
    name: str
    fmt: str
    out: str                      # "f32" or "bf16"
    dist: str
    shapes: Tuple[Tuple[int, int, int], ...]
    batch: int = 0


# The synthetic workloads, numbered 1..5 (value recipes and shapes as named;
# workload 5 has two parts: one 8192^3 product and a batch of 64 products,
# the batch drawn with shape index 1).
WORKLOADS = (
    Workload(1, "bf16-256cube-f32", "bf16", "f32", "uniform", ((256, 256, 256),)),
    Workload(2, "bf16-4096cube-bf16out", "bf16", "bf16", "normal", ((4096, 4096, 4096),)),
    Workload(3, "bf16-ragged-f32", "bf16", "f32", "uniform",
             ((4000, 4000, 4000), (4097, 4095, 4104), (1000, 3000, 777))),
    Workload(4, "bf16-splitk-f32", "bf16", "f32", "normal_sqrtk",
             ((256, 256, 65536), (128, 512, 131072), (64, 64, 262144))),
    Workload(5, "e4m3-8192cube-f32", "e4m3", "f32", "normal", ((8192, 8192, 8192),)),
    Workload(5, "e4m3-batch64-f32", "e4m3", "f32", "normal", ((512, 1024, 4096),), batch=64),
)


def workload_operands(w: Workload, shape_index: int = 0) -> Operands:
    M, N, K = w.shapes[shape_index]
    si = shape_index + (1 if w.batch else 0)
    return make_operands(M, N, K, w.fmt, w.dist, seed_for(w.index, si, 0),
                         seed_for(w.index, si, 1), batch=w.batch)
