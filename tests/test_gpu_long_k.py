"""GPU parity at long K: every product tile's LDS ring wraps many times.

The ring depth is the lever the page "Grid 24 is not headroom" names once
occupancy is gone (section "What is left when occupancy is gone"), and
split-K cuts K into slices that are summed afterwards (page "10. Tensor
Cores, shapes, and tile alignment", section "When shape alone can't fix
wave efficiency").  A stale or skipped ring stage, a slice boundary that
drops or repeats a K-tile, or a unit that starts on the previous unit's ring
changes the sum by a few K-tiles' worth of terms, which a tolerance scaled by
K cannot see at large K.  Here every input is an integer in {-1, 0, 1}
(block-scaled formats: E8M0 scales 2^-2 .. 2^2), so every partial sum is exact
in binary32 in any order and the device must reproduce the oracle bit for bit:

* K gives 64 K-tiles per unit (bf16 4096, 8-bit 8192, FP6 8192, FP4 16384),
  so the deepest ring (8 stages) wraps 8 times and each of 3 split-K slices
  still holds 21 K-tiles, i.e. at least stages + 2;
* every product tile, in every operand-format instantiation it has;
* one workgroup per unit, a uniform 3-way split, a persistent grid of one
  compute unit's resident groups (every workgroup runs several whole units
  in turn on the same ring), and a persistent grid whose partial last round
  is split along K.
"""
import numpy as np
import pytest

from dense_tiled_gemm_fp8_amd import gemm355 as g
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

K_OF_CLASS = {0: 4096, 1: 8192, 2: 8192, 3: 16384, 4: 8192}
M, N = 300, 520

CASES = []
for _t in range(g.gemm355_num_tiles()):
    _info = g.gemm355_tile_info(_t)
    if _info["op"] != 0:
        continue
    for _fmt in H.CLASS_FMTS[_info["dtype_class"]]:
        CASES.append((_t, _fmt))

_REF = {}


def _ops_and_ref(fmt, cls):
    if fmt not in _REF:
        K = K_OF_CLASS[cls]
        ops = H.exact_ops(M, N, K, fmt, 4100 + cls)
        C_ref, _ = H.oracle_full(ops, alpha=1.0)
        # exact in binary32: every sum is an integer multiple of 2^-4 below 2^24
        assert np.all(np.abs(C_ref) < 2.0 ** 20) and np.array_equal(C_ref, C_ref.astype(np.float32))
        _REF[fmt] = (ops, C_ref, H.dev(ops.A), H.dev(ops.B))
    return _REF[fmt]


@pytest.mark.parametrize("tile,fmt", CASES)
def test_long_k_exact_every_tile(tile, fmt):
    info = g.gemm355_tile_info(tile)
    ops, C_ref, A_dev, B_dev = _ops_and_ref(fmt, info["dtype_class"])
    nK = ops.K // info["T_K"]
    assert nK >= 3 * (info["stages"] + 2), (nK, info)
    # plans only inspect pointers (alignment, overlap): C's is a placeholder
    kw = dict(M=M, N=N, K=ops.K, A=A_dev, B=B_dev, C=0x200000000000, dtype=H.out_dtype(fmt, "f32"), tile=tile,
              block_scale_a=0x4000 if ops.mx else None, block_scale_b=0x8000 if ops.mx else None)
    tail_cus = H.split_tail_cus(kw)
    knobs = [dict(split_k=1, persistent=0), dict(split_k=3, persistent=0),
             dict(split_k=1, persistent=1, cus=1)]
    if tail_cus is not None:
        knobs.append(dict(split_k=1, persistent=1, cus=tail_cus))
    for kn in knobs:
        p = g.gemm355_plan(g.make_args(**dict(kw, **kn)))
        H.say("long K", fmt, "tile", tile, "K", ops.K, kn, "units", p["units"], "grid", p["grid"],
              "split", p["split"], "tail", p["tail_tiles"], p["tail_split"])
        C = H.run(ops, out="f32", tile=tile, A_dev=A_dev, B_dev=B_dev, **kn)
        if not np.array_equal(C, C_ref):
            bad = np.argwhere(C != C_ref)
            raise AssertionError("%s tile %d %s: %d of %d outputs differ; first %s gpu %s ref %s" % (
                fmt, tile, kn, len(bad), C.size, bad[:3].tolist(), [C[tuple(i)] for i in bad[:3]],
                [C_ref[tuple(i)] for i in bad[:3]]))
