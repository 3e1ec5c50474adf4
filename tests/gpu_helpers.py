"""Helpers for the GPU parity tests: move raw operand codes to the device,
call libgemm355 through its C ABI, bring C back, compare with the oracle.

Tolerances (per element, W = |alpha| sum_k |a_ik b_kj| from the oracle):
  bf16 inputs:             |C_gpu - C_ref| <= 1e-3 W + 1e-6
  8-bit (E4M3, E5M2) inputs, with or without block scales:
                           |C_gpu - C_ref| <= 2e-2 W
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from dense_tiled_gemm_fp8_amd import gemm355 as g
from dense_tiled_gemm_fp8_amd import inputs
from oracle import mx as mx_oracle
from oracle import reference as oracle

TOL = {"bf16": (1e-3, 1e-6), "e4m3": (2e-2, 0.0), "e5m2": (2e-2, 0.0), "e4m3e5m2": (2e-2, 0.0),
       "mxe4m3": (2e-2, 0.0), "mxe5m2": (2e-2, 0.0), "mxe4m3e5m2": (2e-2, 0.0), "mxfp4": (2e-2, 0.0),
       "mxfp6e2m3": (2e-2, 0.0), "mxfp6e3m2": (2e-2, 0.0)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(codes: np.ndarray) -> torch.Tensor:
    """Raw codes -> device tensor holding the same bytes."""
    c = np.ascontiguousarray(codes)
    if c.dtype == np.uint16:
        t = torch.from_numpy(c.view(np.int16))
    else:
        t = torch.from_numpy(c.view(np.uint8))
    return t.to("cuda")


def out_dtype(fmt: str, out: str) -> int:
    table = {"bf16": (g.BF16_F32, g.BF16_BF16), "e4m3": (g.E4M3_F32, g.E4M3_BF16),
             "e5m2": (g.E5M2_F32, g.E5M2_BF16), "e4m3e5m2": (g.E4M3_E5M2_F32, g.E4M3_E5M2_BF16),
             "mxe4m3": (g.MXE4M3_F32, g.MXE4M3_BF16), "mxe5m2": (g.MXE5M2_F32, g.MXE5M2_BF16),
             "mxe4m3e5m2": (g.MXE4M3_E5M2_F32, g.MXE4M3_E5M2_BF16), "mxfp4": (g.MXFP4_F32, g.MXFP4_BF16),
             "mxfp6e2m3": (g.MXFP6_E2M3_F32, g.MXFP6_E2M3_BF16), "mxfp6e3m2": (g.MXFP6_E3M2_F32, g.MXFP6_E3M2_BF16)}
    return table[fmt][1 if out == "bf16" else 0]


def empty_c(batch: int, M: int, N: int, out: str, fill: float = float("nan")) -> torch.Tensor:
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    shape = (batch, M, N) if batch > 1 else (M, N)
    return torch.full(shape, fill, dtype=dt, device="cuda")


def run(ops: inputs.Operands, out: str = "f32", split_k: int = 0, persistent: int = -1,
        tile: int = -1, layout: int = g.A_ROW_B_COL, A_dev=None, B_dev=None, lda=None, ldb=None,
        scales: bool = True, workspace=None, C=None, cus: int = 0) -> np.ndarray:
    """Run one (batched) product on the device in the storage convention of
    the inputs module (A row-major M x K, B column-major given as N x K)."""
    M, N, K, batch = ops.M, ops.N, ops.K, ops.batch
    A_dev = dev(ops.A) if A_dev is None else A_dev
    B_dev = dev(ops.B) if B_dev is None else B_dev
    if C is None:
        C = empty_c(batch, M, N, out)
    sa = sb = None
    if scales and ops.fmt != "bf16" and not ops.mx:
        sa = torch.tensor(ops.scale_a, dtype=torch.float32, device="cuda")
        sb = torch.tensor(ops.scale_b, dtype=torch.float32, device="cuda")
    bsa = bsb = None
    if ops.mx:
        bsa, bsb = dev(ops.bsa), dev(ops.bsb)
    ws = None
    args = g.make_args(M, N, K, A=A_dev, lda=lda, B=B_dev, ldb=ldb, C=C, dtype=out_dtype(ops.fmt, out),
                       layout=layout, batch=batch, stride_a=M * K, stride_b=N * K, stride_c=M * N,
                       scale_a=sa, scale_b=sb, split_k=split_k, persistent=persistent, tile=tile,
                       block_scale_a=bsa, block_scale_b=bsb, cus=cus)
    if workspace == "caller":
        p = g.gemm355_plan(args)
        if p["workspace_bytes"]:
            ws = torch.empty(p["workspace_bytes"], dtype=torch.uint8, device="cuda")
            args.workspace = ws.data_ptr()
            args.workspace_bytes = p["workspace_bytes"]
    g.gemm355_gemm_ex(args)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def alpha_of(ops: inputs.Operands, bi: int = 0) -> float:
    if ops.fmt != "bf16" and not ops.mx:
        return float(np.float32(ops.scale_a[bi]) * np.float32(ops.scale_b[bi]))
    return 1.0


def oracle_full(ops: inputs.Operands, bi: int = 0, alpha=None):
    A = ops.A[bi] if ops.A.ndim == 3 else ops.A
    B = ops.B[bi] if ops.B.ndim == 3 else ops.B
    if alpha is None:
        alpha = alpha_of(ops, bi)
    if ops.mx:
        bsa = ops.bsa[bi] if ops.bsa.ndim == 3 else ops.bsa
        bsb = ops.bsb[bi] if ops.bsb.ndim == 3 else ops.bsb
        return mx_oracle.gemm(A, bsa, B, bsb, ops.fmt_a, ops.fmt_b, alpha=alpha)
    return oracle.gemm(ops.M, ops.N, ops.K, A.reshape(-1), ops.K, B.reshape(-1), ops.K, alpha=alpha,
                       **fmt_kw(ops))


def oracle_entries(ops: inputs.Operands, rows, cols, bi: int = 0):
    A = ops.A[bi] if ops.A.ndim == 3 else ops.A
    B = ops.B[bi] if ops.B.ndim == 3 else ops.B
    if ops.mx:
        bsa = ops.bsa[bi] if ops.bsa.ndim == 3 else ops.bsa
        bsb = ops.bsb[bi] if ops.bsb.ndim == 3 else ops.bsb
        return mx_oracle.gemm_entries(A, bsa, B, bsb, rows, cols, ops.fmt_a, ops.fmt_b, alpha=alpha_of(ops, bi))
    return oracle.gemm_entries(ops.K, A.reshape(-1), ops.K, B.reshape(-1), ops.K, rows, cols,
                               alpha=alpha_of(ops, bi), **fmt_kw(ops))


def fmt_kw(ops: inputs.Operands):
    """The oracle's format arguments for the operands' codes."""
    if ops.fmt == "bf16":
        return {}
    return {"fmt_a": ops.fmt_a, "fmt_b": ops.fmt_b}


def check(C_gpu: np.ndarray, C_ref: np.ndarray, W: np.ndarray, fmt: str, what: str = ""):
    rel, absol = TOL[fmt]
    err = np.abs(C_gpu - C_ref)
    bound = rel * W + absol
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outside tolerance; first %s: gpu %s ref %s W %s" % (
            what, int(bad.sum()), bad.size, idx.tolist(),
            [C_gpu[tuple(i)] for i in idx], [C_ref[tuple(i)] for i in idx], [W[tuple(i)] for i in idx]))


def sample_positions(M: int, N: int, n: int, seed: int):
    """Random positions plus the four corners and the last row/column
    stretches (ragged edges)."""
    r = np.random.Generator(np.random.PCG64(seed))
    rows = list(r.integers(0, M, n))
    cols = list(r.integers(0, N, n))
    for (i, j) in [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]:
        rows.append(i)
        cols.append(j)
    edge = min(64, N)
    rows += [M - 1] * edge
    cols += list(range(N - edge, N))
    edge = min(64, M)
    rows += list(range(M - edge, M))
    cols += [N - 1] * edge
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


# operand formats of each input class of the tile table
CLASS_FMTS = {0: ("bf16",), 1: ("e4m3", "e5m2", "e4m3e5m2"), 2: ("mxe4m3", "mxe5m2", "mxe4m3e5m2"),
              3: ("mxfp4",), 4: ("mxfp6e2m3", "mxfp6e3m2")}


def elem_formats(fmt: str):
    """(A's, B's) element format names of a dtype name."""
    if fmt == "bf16":
        return "bf16", "bf16"
    if fmt.startswith("mxfp6"):
        return fmt[5:], fmt[5:]
    if fmt == "mxfp4":
        return "e2m1", "e2m1"
    base = fmt[2:] if fmt.startswith("mx") else fmt
    if base == "e4m3e5m2":
        return "e4m3", "e5m2"
    return base, base


def exact_ops(M: int, N: int, K: int, fmt: str, seed: int, batch: int = 0, lo: int = -1, hi: int = 1,
              scale_lo: int = 125, scale_hi: int = 129) -> inputs.Operands:
    """Integer elements in [lo, hi] in any input format; block-scaled formats
    get E8M0 scales in [scale_lo, scale_hi] (2^-2 .. 2^2 by default).  With
    |products| <= 2^4 and K * 2^4 * max|a b| below 2^20, every partial sum
    is a multiple of 2^-4 below 2^24 in magnitude, i.e. exact in binary32 in
    any summation order."""
    ga, gb = inputs.rng(seed), inputs.rng(seed + 1)
    fa, fb = elem_formats(fmt)
    nb = max(batch, 1)
    A = np.stack([inputs.small_int_codes(ga, (M, K), fa, lo, hi) for _ in range(nb)])
    B = np.stack([inputs.small_int_codes(gb, (N, K), fb, lo, hi) for _ in range(nb)])
    sa = sb = None
    if fmt.startswith("mx"):
        sa = np.stack([ga.integers(scale_lo, scale_hi + 1, size=(M, K // 32)).astype(np.uint8)
                       for _ in range(nb)])
        sb = np.stack([gb.integers(scale_lo, scale_hi + 1, size=(N, K // 32)).astype(np.uint8)
                       for _ in range(nb)])
    if not batch:
        A, B = A[0], B[0]
        if sa is not None:
            sa, sb = sa[0], sb[0]
    return inputs.Operands(M, N, K, fmt, A, B, [1.0] * nb, [1.0] * nb, (seed, seed + 1), sa, sb)


def split_tail_cus(args_kw: dict, limit: int = 16):
    """The smallest planning CU count (1 .. limit) whose persistent plan for
    these arguments splits a partial last round along K while some
    workgroup runs more than one unit; None if there is none."""
    for cus in range(1, limit + 1):
        a = g.make_args(**dict(args_kw, cus=cus, persistent=1, split_k=1))
        p = g.gemm355_plan(a)
        if p["tail_tiles"] > 0 and p["units"] > p["grid"] and p["units"] - p["tail_tiles"] * p["tail_split"] > 0:
            return cus
    return None
