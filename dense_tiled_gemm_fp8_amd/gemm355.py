"""ctypes binding of libgemm355 (include/gemm355.h): argument marshalling only.

Every function here has the name of the C entry point it wraps and does no
arithmetic of its own: all work runs in the library's HIP kernels.  Pointers
may be passed as torch tensors (their ``data_ptr()``) or plain integers;
``stream=None`` means torch's current stream on the current device.

Importing this module loads ``libgemm355.so`` and raises ImportError if it
has not been built (``python -m dense_tiled_gemm_fp8_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Any, Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm355.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libgemm355.so is not built; run python -m dense_tiled_gemm_fp8_amd.build")
# One HIP runtime per process: PyTorch's ROCm wheels carry their own
# libamdhip64, which they load under a name the dynamic loader does not match
# to a runtime already loaded from the system ROCm, so loading this library
# first would leave two runtimes (and torch's device memory foreign to the
# one this library launches on).  Loaded after torch, the library binds to
# torch's runtime.
try:
    import torch  # noqa: F401
except ImportError:   # no PyTorch in the process: the system runtime is the only one
    pass
_lib = ctypes.CDLL(LIB_PATH)

# status codes
OK, EINVAL, EALIGN, EUNSUPPORTED, ENOMEM, EHIP, ETOOBIG = range(7)
# dtypes (input -> output)
(BF16_F32, BF16_BF16, E4M3_F32, E4M3_BF16, E5M2_F32, E5M2_BF16, E4M3_E5M2_F32,
 E4M3_E5M2_BF16, MXE4M3_F32, MXE4M3_BF16, MXE5M2_F32, MXE5M2_BF16, MXE4M3_E5M2_F32,
 MXE4M3_E5M2_BF16, MXFP4_F32, MXFP4_BF16, MXFP6_E2M3_F32, MXFP6_E2M3_BF16, MXFP6_E3M2_F32,
 MXFP6_E3M2_BF16) = range(20)
# 8-bit formats and source types of the quantiser
FP8_E4M3, FP8_E5M2 = range(2)
SRC_F32, SRC_BF16 = range(2)
# layouts
A_ROW_B_COL, A_ROW_B_ROW, A_COL_B_COL, A_COL_B_ROW = range(4)

_i64, _i32, _vp, _f64, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double, ctypes.c_size_t


class gemm355_args(ctypes.Structure):
    _fields_ = [
        ("M", _i64), ("N", _i64), ("K", _i64),
        ("A", _vp), ("lda", _i64), ("stride_a", _i64),
        ("B", _vp), ("ldb", _i64), ("stride_b", _i64),
        ("C", _vp), ("ldc", _i64), ("stride_c", _i64),
        ("batch", _i64),
        ("scale_a", _vp), ("scale_b", _vp),
        ("dtype", ctypes.c_int), ("layout", ctypes.c_int),
        ("split_k", _i32), ("persistent", _i32), ("tile", _i32), ("cus", _i32),
        ("workspace", _vp), ("workspace_bytes", _sz),
        ("unit_stamps", _vp),
        ("block_scale_a", _vp), ("block_scale_b", _vp),
    ]


class gemm355_plan_t(ctypes.Structure):
    _fields_ = [
        ("tile", _i32), ("T_M", _i32), ("T_N", _i32), ("T_K", _i32),
        ("stages", _i32), ("waves", _i32), ("lds_bytes", _i32), ("vgpr_budget", _i32),
        ("S", _i32), ("b", _i32),
        ("G", _i64), ("nK", _i64), ("M_pad", _i64), ("N_pad", _i64), ("K_pad", _i64),
        ("split", _i32), ("persistent", _i32),
        ("tail_tiles", _i64), ("tail_split", _i32), ("repack", _i32),
        ("units", _i64), ("grid", _i64),
        ("eta_wave_num", _i64), ("eta_wave_den", _i64),
        ("eta_pad_num", _i64), ("eta_pad_den", _i64),
        ("eta_sched_num", _i64), ("eta_sched_den", _i64),
        ("workspace_bytes", _sz),
        ("model_seconds", ctypes.c_double),
        ("model_mfma_peak_seconds", ctypes.c_double), ("model_mfma_eff", ctypes.c_double),
        ("model_bytes", ctypes.c_double), ("model_spread", ctypes.c_double),
        ("model_stream_eff", ctypes.c_double), ("model_copy_seconds", ctypes.c_double),
        ("model_fixed_seconds", ctypes.c_double), ("model_units_in_turn", _i64),
    ]


class gemm355_conv_args(ctypes.Structure):
    _fields_ = [
        ("N", _i64), ("H", _i64), ("W", _i64), ("C", _i64),
        ("K", _i64), ("R", _i64), ("S", _i64),
        ("pad_h", _i64), ("pad_w", _i64), ("stride_h", _i64), ("stride_w", _i64),
        ("dil_h", _i64), ("dil_w", _i64),
        ("x", _vp), ("w", _vp), ("y", _vp),
        ("dtype", ctypes.c_int),
        ("split_k", _i32), ("persistent", _i32), ("tile", _i32), ("cus", _i32),
        ("workspace", _vp), ("workspace_bytes", _sz),
    ]


_lib.gemm355_gemm.restype = ctypes.c_int
_lib.gemm355_gemm.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                              ctypes.c_int, ctypes.c_int, _i32, _i32, _vp]
_lib.gemm355_gemm_ex.restype = ctypes.c_int
_lib.gemm355_gemm_ex.argtypes = [ctypes.POINTER(gemm355_args), _vp]
_lib.gemm355_gemm_noalloc.restype = ctypes.c_int
_lib.gemm355_gemm_noalloc.argtypes = [ctypes.POINTER(gemm355_args), _vp]
_lib.gemm355_plan.restype = ctypes.c_int
_lib.gemm355_plan.argtypes = [ctypes.POINTER(gemm355_args), ctypes.POINTER(gemm355_plan_t)]
_lib.gemm355_eta_wave.restype = _f64
_lib.gemm355_eta_wave.argtypes = [_i64, _i32, _i32]
_lib.gemm355_eta_pad.restype = _f64
_lib.gemm355_eta_pad.argtypes = [_i64] * 6
_lib.gemm355_kslice.restype = ctypes.c_int
_lib.gemm355_kslice.argtypes = [_i64, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
_lib.gemm355_unit.restype = ctypes.c_int
_lib.gemm355_unit.argtypes = [ctypes.POINTER(gemm355_args), _i64] + [ctypes.POINTER(_i64)] * 5
_lib.gemm355_num_tiles.restype = _i32
_lib.gemm355_num_tiles.argtypes = []
_lib.gemm355_tile_info.restype = ctypes.c_int
_lib.gemm355_tile_info.argtypes = [_i32] + [ctypes.POINTER(_i32)] * 10
_lib.gemm355_tile_occupancy.restype = ctypes.c_int
_lib.gemm355_tile_occupancy.argtypes = [_i32, ctypes.POINTER(_i32)]
_lib.gemm355_quantize.restype = ctypes.c_int
_lib.gemm355_quantize.argtypes = [_vp, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]
_lib.gemm355_conv2d.restype = ctypes.c_int
_lib.gemm355_conv2d.argtypes = [ctypes.POINTER(gemm355_conv_args), _vp]
_lib.gemm355_conv2d_plan.restype = ctypes.c_int
_lib.gemm355_conv2d_plan.argtypes = [ctypes.POINTER(gemm355_conv_args), ctypes.POINTER(gemm355_plan_t)]
_lib.gemm355_conv2d_out_size.restype = ctypes.c_int
_lib.gemm355_conv2d_out_size.argtypes = [ctypes.POINTER(gemm355_conv_args), ctypes.POINTER(_i64),
                                         ctypes.POINTER(_i64)]
_lib.gemm355_set_scratch_limit.restype = ctypes.c_int
_lib.gemm355_set_scratch_limit.argtypes = [ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
_lib.gemm355_status_string.restype = ctypes.c_char_p
_lib.gemm355_status_string.argtypes = [ctypes.c_int]

EXPORTED = ("gemm355_gemm", "gemm355_gemm_ex", "gemm355_gemm_noalloc",
            "gemm355_plan", "gemm355_eta_wave",
            "gemm355_eta_pad", "gemm355_kslice", "gemm355_unit", "gemm355_num_tiles",
            "gemm355_tile_info", "gemm355_tile_occupancy", "gemm355_quantize",
            "gemm355_conv2d", "gemm355_conv2d_plan", "gemm355_conv2d_out_size", "gemm355_set_scratch_limit",
            "gemm355_status_string")


class Gemm355Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, gemm355_status_string(status), status))


def _ptr(x: Any) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream: Any) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return int(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int, where: str) -> None:
    if status != OK:
        raise Gemm355Error(status, where)


def gemm355_status_string(status: int) -> str:
    return _lib.gemm355_status_string(status).decode()


def gemm355_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, layout=A_ROW_B_COL, split_k=0,
                 persistent=-1, stream=None) -> None:
    _check(_lib.gemm355_gemm(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, dtype, layout,
                             split_k, persistent, _stream(stream)), "gemm355_gemm")


def make_args(M, N, K, A=None, lda=None, B=None, ldb=None, C=None, ldc=None, dtype=BF16_F32,
              layout=A_ROW_B_COL, batch=1, stride_a=0, stride_b=0, stride_c=0, scale_a=None,
              scale_b=None, split_k=0, persistent=-1, tile=-1, cus=0, workspace=None,
              workspace_bytes=0, unit_stamps=None, block_scale_a=None,
              block_scale_b=None) -> gemm355_args:
    """Fill a gemm355_args; leading dimensions default to the packed ones."""
    a_row = layout in (A_ROW_B_COL, A_ROW_B_ROW)
    b_col = layout in (A_ROW_B_COL, A_COL_B_COL)
    if lda is None:
        lda = max(1, K if a_row else M)
    if ldb is None:
        ldb = max(1, K if b_col else N)
    if ldc is None:
        ldc = max(1, N)
    return gemm355_args(M, N, K, _ptr(A), lda, stride_a, _ptr(B), ldb, stride_b, _ptr(C), ldc,
                        stride_c, batch, _ptr(scale_a), _ptr(scale_b), dtype, layout, split_k,
                        persistent, tile, cus, _ptr(workspace), workspace_bytes, _ptr(unit_stamps),
                        _ptr(block_scale_a), _ptr(block_scale_b))


def gemm355_gemm_ex(args: gemm355_args, stream=None) -> None:
    _check(_lib.gemm355_gemm_ex(ctypes.byref(args), _stream(stream)), "gemm355_gemm_ex")


def gemm355_gemm_noalloc(args: gemm355_args, stream=None) -> None:
    _check(_lib.gemm355_gemm_noalloc(ctypes.byref(args), _stream(stream)), "gemm355_gemm_noalloc")


def gemm355_plan(args: gemm355_args) -> Dict[str, int]:
    out = gemm355_plan_t()
    _check(_lib.gemm355_plan(ctypes.byref(args), ctypes.byref(out)), "gemm355_plan")
    return {name: getattr(out, name) for name, _ in gemm355_plan_t._fields_}


def gemm355_eta_wave(G: int, S: int, b: int) -> float:
    return _lib.gemm355_eta_wave(G, S, b)


def gemm355_eta_pad(M: int, N: int, K: int, T_M: int, T_N: int, T_K: int) -> float:
    return _lib.gemm355_eta_pad(M, N, K, T_M, T_N, T_K)


def gemm355_kslice(nK: int, s: int, i: int):
    b, e = _i64(), _i64()
    _check(_lib.gemm355_kslice(nK, s, i, ctypes.byref(b), ctypes.byref(e)), "gemm355_kslice")
    return b.value, e.value


def gemm355_unit(args: gemm355_args, u: int):
    vals = [_i64() for _ in range(5)]
    _check(_lib.gemm355_unit(ctypes.byref(args), u, *[ctypes.byref(v) for v in vals]),
           "gemm355_unit")
    return tuple(v.value for v in vals)   # batch, tile_m, tile_n, kt_begin, kt_end


def gemm355_num_tiles() -> int:
    return _lib.gemm355_num_tiles()


def gemm355_tile_info(tile: int) -> Dict[str, int]:
    vals = [_i32() for _ in range(10)]
    _check(_lib.gemm355_tile_info(tile, *[ctypes.byref(v) for v in vals]), "gemm355_tile_info")
    names = ("dtype_class", "T_M", "T_N", "T_K", "stages", "waves", "lds_bytes", "b_max", "op", "schedule")
    return dict(zip(names, (v.value for v in vals)))


SCRATCH_UNLIMITED = (1 << 64) - 1


def gemm355_set_scratch_limit(nbytes: int) -> int:
    """Cap on library-owned scratch (SCRATCH_UNLIMITED: none); returns the previous cap."""
    prev = ctypes.c_uint64()
    _check(_lib.gemm355_set_scratch_limit(nbytes, ctypes.byref(prev)), "gemm355_set_scratch_limit")
    return prev.value


def gemm355_tile_occupancy(tile: int) -> int:
    n = _i32()
    _check(_lib.gemm355_tile_occupancy(tile, ctypes.byref(n)), "gemm355_tile_occupancy")
    return n.value


def make_conv_args(N, H, W, C, K, R, S, x=None, w=None, y=None, pad_h=0, pad_w=0, stride_h=1,
                   stride_w=1, dil_h=1, dil_w=1, dtype=BF16_F32, split_k=0, persistent=-1, tile=-1,
                   cus=0, workspace=None, workspace_bytes=0) -> gemm355_conv_args:
    return gemm355_conv_args(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w,
                             _ptr(x), _ptr(w), _ptr(y), dtype, split_k, persistent, tile, cus,
                             _ptr(workspace), workspace_bytes)


def gemm355_conv2d(args: gemm355_conv_args, stream=None) -> None:
    _check(_lib.gemm355_conv2d(ctypes.byref(args), _stream(stream)), "gemm355_conv2d")


def gemm355_conv2d_out_size(args: gemm355_conv_args):
    """(P, Q): the output extent the library gives this convolution."""
    P, Q = _i64(), _i64()
    _check(_lib.gemm355_conv2d_out_size(ctypes.byref(args) if args is not None else None, ctypes.byref(P),
                                        ctypes.byref(Q)), "gemm355_conv2d_out_size")
    return P.value, Q.value


def gemm355_conv2d_plan(args: gemm355_conv_args) -> Dict[str, int]:
    out = gemm355_plan_t()
    _check(_lib.gemm355_conv2d_plan(ctypes.byref(args) if args is not None else None, ctypes.byref(out)),
           "gemm355_conv2d_plan")
    return {name: getattr(out, name) for name, _ in gemm355_plan_t._fields_}


def gemm355_quantize(x, n, batch, src, fmt, q, scale, stream=None) -> None:
    """Per-tensor scaling of `batch` tensors of n elements to 8-bit codes q,
    dequantisation factors into scale[batch] (device pointers or tensors)."""
    _check(_lib.gemm355_quantize(_ptr(x), n, batch, src, fmt, _ptr(q), _ptr(scale), _stream(stream)),
           "gemm355_quantize")
