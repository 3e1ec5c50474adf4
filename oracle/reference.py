"""ctypes wrapper around ``gemm_oracle.c`` (the binary64 triple-loop product).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.

The product follows the problem statement and the FLOPs equation in section
"Shape the operation" of page "10. Tensor Cores, shapes, and tile alignment":
C = A B with the K-term dot product written out, decoded to binary64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_BF16 = 0
FMT_E4M3 = 1
FMT_E5M2 = 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP, -O2, strict IEEE binary64)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            i64, vp, ci, cd = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
            lib.oracle_gemm.restype = i64
            lib.oracle_gemm.argtypes = [i64, i64, i64, vp, i64, ci, vp, i64, ci, ci, ci, cd, vp, vp]
            lib.oracle_gemm_entries.restype = i64
            lib.oracle_gemm_entries.argtypes = [i64, vp, i64, ci, vp, i64, ci, ci, ci, cd,
                                                i64, vp, vp, vp, vp]
            lib.oracle_threads.restype = ci
            lib.oracle_decode_bf16.restype = cd
            lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
            lib.oracle_decode_e4m3.restype = cd
            lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
            lib.oracle_decode_e5m2.restype = cd
            lib.oracle_decode_e5m2.argtypes = [ctypes.c_uint8]
            _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_threads())


def _fmt_of(codes: np.ndarray, name: Optional[str]) -> int:
    """Element format of a code array: uint16 is bf16; uint8 is an 8-bit
    float, E4M3 unless ``name`` says "e5m2"."""
    if codes.dtype == np.uint16:
        if name not in (None, "bf16"):
            raise TypeError("uint16 codes are bf16")
        return FMT_BF16
    if codes.dtype == np.uint8:
        if name in (None, "e4m3"):
            return FMT_E4M3
        if name == "e5m2":
            return FMT_E5M2
        raise TypeError("uint8 codes are e4m3 or e5m2, not %r" % (name,))
    raise TypeError("oracle inputs are raw codes: uint16 (bf16) or uint8 (E4M3 / E5M2)")


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def gemm(M: int, N: int, K: int, A: np.ndarray, lda: int, B: np.ndarray, ldb: int,
         a_colmajor: bool = False, b_rowmajor: bool = False, alpha: float = 1.0,
         with_w: bool = True, return_macs: bool = False, fmt_a: Optional[str] = None,
         fmt_b: Optional[str] = None):
    """Full product.  ``A`` and ``B`` are flat code arrays addressed with
    ``lda``/``ldb`` as described in ``gemm_oracle.c``; 8-bit codes are E4M3
    unless ``fmt_a`` / ``fmt_b`` name "e5m2".  Returns ``(C, W)`` as
    binary64 M x N arrays (``W`` is None if ``with_w`` is False), plus the
    multiply-add count if ``return_macs``."""
    fa, fb = _fmt_of(A, fmt_a), _fmt_of(B, fmt_b)
    if (fa == FMT_BF16) != (fb == FMT_BF16):
        raise TypeError("A and B must both be bf16 or both 8-bit")
    A = np.ascontiguousarray(A).reshape(-1)
    B = np.ascontiguousarray(B).reshape(-1)
    C = np.zeros((max(M, 0), max(N, 0)), dtype=np.float64)
    W = np.zeros_like(C) if with_w else None
    if M > 0 and N > 0:
        macs = _load().oracle_gemm(M, N, K, _ptr(A), lda, int(a_colmajor), _ptr(B), ldb,
                                   int(b_rowmajor), fa, fb, float(alpha), _ptr(C),
                                   _ptr(W) if W is not None else None)
        if macs < 0:
            raise MemoryError("oracle scratch allocation failed")
    else:
        macs = 0
    if return_macs:
        return C, W, int(macs)
    return C, W


def gemm_entries(K: int, A: np.ndarray, lda: int, B: np.ndarray, ldb: int,
                 rows: np.ndarray, cols: np.ndarray, a_colmajor: bool = False,
                 b_rowmajor: bool = False, alpha: float = 1.0, fmt_a: Optional[str] = None,
                 fmt_b: Optional[str] = None):
    """Selected entries (rows[t], cols[t]) of the same product, each its own
    K-term dot product.  Returns ``(c, w)`` binary64 vectors."""
    fa, fb = _fmt_of(A, fmt_a), _fmt_of(B, fmt_b)
    if (fa == FMT_BF16) != (fb == FMT_BF16):
        raise TypeError("A and B must both be bf16 or both 8-bit")
    A = np.ascontiguousarray(A).reshape(-1)
    B = np.ascontiguousarray(B).reshape(-1)
    ii = np.ascontiguousarray(rows, dtype=np.int64)
    jj = np.ascontiguousarray(cols, dtype=np.int64)
    c = np.zeros(ii.shape[0], dtype=np.float64)
    w = np.zeros_like(c)
    if ii.shape[0]:
        _load().oracle_gemm_entries(K, _ptr(A), lda, int(a_colmajor), _ptr(B), ldb,
                                    int(b_rowmajor), fa, fb, float(alpha), ii.shape[0],
                                    _ptr(ii), _ptr(jj), _ptr(c), _ptr(w))
    return c, w


def decode_bf16(codes: np.ndarray) -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_decode_bf16(int(c)) for c in np.asarray(codes).reshape(-1)])


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_decode_e4m3(int(c)) for c in np.asarray(codes).reshape(-1)])


def decode_e5m2(codes: np.ndarray) -> np.ndarray:
    lib = _load()
    return np.array([lib.oracle_decode_e5m2(int(c)) for c in np.asarray(codes).reshape(-1)])
