"""GPU parity on seeded random cases: a random input format (bf16, the
8-bit formats and their mix, MXFP8, MXFP6, MXFP4), shape, batch, tile of the
table (or the planner's choice) and split / persistence knob, with small
integer inputs and E8M0 scales of 2^-2 .. 2^2, so that every sum is exact in
binary32 in any order: each output must equal the oracle's bit for bit.  The
fixed-shape tests pin the named paths; this sweep looks for the corner a
fixed list misses (a ragged edge of one tile meeting a split tail, a short K
in a deep ring, a batch stride on a forced tile)."""
import random

import numpy as np
import pytest

from dense_tiled_gemm_fp8_amd import gemm355 as g
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CLASS = {"bf16": 0, "e4m3": 1, "e5m2": 1, "e4m3e5m2": 1, "mxe4m3": 2, "mxfp4": 3, "mxfp6e2m3": 4}
TILES = {}
for _t in range(g.gemm355_num_tiles()):
    _i = g.gemm355_tile_info(_t)
    if _i["op"] == 0:
        TILES.setdefault(_i["dtype_class"], []).append(_t)

KNOBS = [dict(), dict(split_k=1, persistent=0), dict(split_k=1, persistent=1), dict(split_k=2),
         dict(split_k=3, persistent=1), dict(split_k=6), dict(persistent=1, cus=7), dict(cus=13)]


@pytest.mark.parametrize("block", range(4))
def test_random_cases_exact(block):
    rnd = random.Random(1000 + block)
    for case in range(30):
        fmt = rnd.choice(list(CLASS))
        M, N = rnd.randint(1, 520), rnd.randint(1, 520)
        if fmt.startswith("mx"):
            step = 256 if fmt == "mxfp4" else 128
            K = step * rnd.randint(1, 1536 // step)
        else:
            K = rnd.randint(1, 1600)
        batch = rnd.choice([0, 0, 2, 3])
        tile = rnd.choice(TILES[CLASS[fmt]] + [-1, -1])
        knobs = rnd.choice(KNOBS)
        seed = 50000 + 100 * block + case
        ops = H.exact_ops(M, N, K, fmt, seed, batch=batch)
        what = "case %d.%d: %s M=%d N=%d K=%d batch=%d tile=%d %s" % (block, case, fmt, M, N, K, batch, tile, knobs)
        H.say(what)
        C = H.run(ops, out="f32", tile=tile, **knobs)
        Cb = C if batch else C[None]
        for bi in range(max(batch, 1)):
            ref, _ = H.oracle_full(ops, bi, alpha=1.0)
            assert np.array_equal(Cb[bi], ref), what
