"""GPU parity for block-scaled ("microscaled") 8-bit products: the
precision-table row after the FP8 pair on page "The Tensor Core", read as
the OCP MX format (32-value blocks along K, E8M0 scales).

* element by element against oracle/mx.py (binary64) within 2e-2 * W on
  ragged shapes, every block-scaled tile, the three operand-format pairs,
  fp32 and bf16 C, split-K, the persistent grid, batches and the other
  operand layouts;
* bit-exact on small integers with scales 2^-2 .. 2^2, where every product
  and partial sum is exact in binary32;
* 4096^3 products on every output;
* a scale that changes inside one K-tile reaches only its own block.
"""
import numpy as np
import pytest
import torch

from dense_tiled_gemm_fp8_amd import gemm355 as g
from dense_tiled_gemm_fp8_amd import inputs
from oracle import mx as omx
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

MX_TILES = [t for t in range(g.gemm355_num_tiles()) if g.gemm355_tile_info(t)["dtype_class"] == 2]
FP4_TILES = [t for t in range(g.gemm355_num_tiles()) if g.gemm355_tile_info(t)["dtype_class"] == 3]
FP6_TILES = [t for t in range(g.gemm355_num_tiles()) if g.gemm355_tile_info(t)["dtype_class"] == 4]


def _bf16_ok(C, C_ref, W, fmt):
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(C_ref), 2.0 ** -126))) - 7)
    return np.all(np.abs(C - C_ref) <= H.TOL[fmt][0] * W + ulp / 2)


@pytest.mark.parametrize("fmt", ["mxe4m3", "mxe5m2", "mxe4m3e5m2"])
@pytest.mark.parametrize("shape", [(300, 520, 256), (257, 129, 384), (70, 90, 128), (1, 1, 128)])
def test_mx_ragged_full(fmt, shape):
    M, N, K = shape
    ops = inputs.make_operands(M, N, K, fmt, "normal", 700 + M + K, 701 + N)
    C_ref, W = H.oracle_full(ops)
    for tile in [-1] + MX_TILES:
        for out in ("f32", "bf16"):
            H.say(fmt, "tile", tile, shape, out)
            C = H.run(ops, out=out, tile=tile)
            if out == "f32":
                H.check(C, C_ref, W, fmt, "%s tile %d %s" % (fmt, tile, shape))
            else:
                assert _bf16_ok(C, C_ref, W, fmt), (fmt, tile, shape)


@pytest.mark.parametrize("shape", [(300, 520, 256), (257, 129, 512), (70, 90, 256), (1, 1, 256)])
def test_mxfp4_ragged_full(shape):
    M, N, K = shape
    ops = inputs.make_operands(M, N, K, "mxfp4", "normal", 800 + M + K, 801 + N)
    C_ref, W = H.oracle_full(ops)
    for tile in [-1] + FP4_TILES:
        for out in ("f32", "bf16"):
            H.say("mxfp4 tile", tile, shape, out)
            C = H.run(ops, out=out, tile=tile)
            if out == "f32":
                H.check(C, C_ref, W, "mxfp4", "mxfp4 tile %d %s" % (tile, shape))
            else:
                assert _bf16_ok(C, C_ref, W, "mxfp4"), (tile, shape)


def _int_ops(M, N, K, fmt, seed, batch=0):
    """Elements in [-4, 4] and scales 125 .. 129 (2^-2 .. 2^2): every
    product is a multiple of 2^-4 of magnitude at most 2^8, so every partial
    sum is exact in binary32 for K <= 2^12."""
    ga, gb = inputs.rng(seed), inputs.rng(seed + 1)
    if fmt.startswith("mxfp6"):
        fa = fb = fmt[5:]
    else:
        fa = "e2m1" if fmt == "mxfp4" else "e5m2" if fmt == "mxe5m2" else "e4m3"
        fb = "e2m1" if fmt == "mxfp4" else "e4m3" if fmt == "mxe4m3" else "e5m2"
    nb = max(batch, 1)
    A = np.stack([inputs.small_int_codes(ga, (M, K), fa) for _ in range(nb)])
    B = np.stack([inputs.small_int_codes(gb, (N, K), fb) for _ in range(nb)])
    sa = np.stack([ga.integers(125, 130, size=(M, K // 32)).astype(np.uint8) for _ in range(nb)])
    sb = np.stack([gb.integers(125, 130, size=(N, K // 32)).astype(np.uint8) for _ in range(nb)])
    if not batch:
        A, B, sa, sb = A[0], B[0], sa[0], sb[0]
    return inputs.Operands(M, N, K, fmt, A, B, [1.0] * nb, [1.0] * nb, (seed, seed + 1), sa, sb)


@pytest.mark.parametrize("fmt", ["mxe4m3", "mxe5m2", "mxe4m3e5m2", "mxfp4", "mxfp6e2m3", "mxfp6e3m2"])
def test_mx_exact_integers_every_tile(fmt):
    M, N, K, batch = 200, 170, 512, 2
    ops = _int_ops(M, N, K, fmt, 81, batch=batch)
    refs = [H.oracle_full(ops, bi)[0] for bi in range(batch)]
    tiles = FP4_TILES if fmt == "mxfp4" else FP6_TILES if fmt.startswith("mxfp6") else MX_TILES
    for tile in tiles:
        for knobs in (dict(split_k=1, persistent=0), dict(split_k=3), dict(persistent=1)):
            H.say(fmt, "ints tile", tile, knobs)
            C = H.run(ops, out="f32", tile=tile, **knobs)
            for bi in range(batch):
                assert np.array_equal(C[bi], refs[bi]), (fmt, tile, knobs, bi)


def test_mx_block_boundaries():
    """One row of A and one column of B with a different scale in each of
    the four blocks of every K-tile: each block's scale multiplies exactly
    its own 32 values (a shifted or swapped block index changes the
    result)."""
    M, N, K = 64, 64, 512
    ops = _int_ops(M, N, K, "mxe4m3", 91)
    ops.bsa[5] = np.tile(np.array([125, 126, 128, 129], dtype=np.uint8), K // 128)
    ops.bsb[9] = np.tile(np.array([129, 125, 127, 128], dtype=np.uint8), K // 128)
    C_ref, _ = H.oracle_full(ops)
    for tile in [-1] + MX_TILES:
        C = H.run(ops, out="f32", tile=tile)
        assert np.array_equal(C, C_ref), tile


def test_mx_per_tensor_scales_and_layouts():
    """Per-tensor scales still multiply the result; the other operand
    layouts are repacked and keep their scales per row of A and column of
    B."""
    M, N, K = 190, 230, 384
    ops = inputs.make_operands(M, N, K, "mxe4m3", "normal", 95, 96)
    C_ref, W = H.oracle_full(ops, alpha=0.375)
    sa = torch.tensor([0.75], dtype=torch.float32, device="cuda")
    sb = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    C = H.empty_c(1, M, N, "f32")
    args = g.make_args(M, N, K, A=H.dev(ops.A), B=H.dev(ops.B), C=C, dtype=g.MXE4M3_F32, scale_a=sa,
                       scale_b=sb, block_scale_a=H.dev(ops.bsa), block_scale_b=H.dev(ops.bsb))
    g.gemm355_gemm_ex(args)
    torch.cuda.synchronize()
    H.check(C.double().cpu().numpy(), C_ref, W, "mxe4m3", "per-tensor scales")
    C_ref1, W1 = H.oracle_full(ops)
    At = np.ascontiguousarray(ops.A.T)          # A column-major: K x M
    Br = np.ascontiguousarray(ops.B.T)          # B row-major: K x N
    for layout, A_dev, B_dev, lda, ldb in ((g.A_COL_B_COL, H.dev(At), H.dev(ops.B), M, K),
                                           (g.A_ROW_B_ROW, H.dev(ops.A), H.dev(Br), K, N),
                                           (g.A_COL_B_ROW, H.dev(At), H.dev(Br), M, N)):
        H.say("layout", layout)
        C = H.run(ops, out="f32", layout=layout, A_dev=A_dev, B_dev=B_dev, lda=lda, ldb=ldb)
        H.check(C, C_ref1, W1, "mxe4m3", "layout %d" % layout)


def test_mx_batch_split_and_persistent():
    M, N, K, batch = 300, 260, 640, 3
    ops = inputs.make_operands(M, N, K, "mxe5m2", "normal", 97, 98, batch=batch)
    refs = [H.oracle_full(ops, bi) for bi in range(batch)]
    for knobs in (dict(), dict(split_k=4), dict(persistent=1), dict(split_k=2, persistent=1),
                  dict(workspace="caller", split_k=5)):
        H.say("mx batch", knobs)
        C = H.run(ops, out="f32", **knobs)
        for bi in range(batch):
            H.check(C[bi], refs[bi][0], refs[bi][1], "mxe5m2", "batch %d %s" % (bi, knobs))


def test_mxfp4_block_boundaries_and_batch():
    """FP4: a different scale in each of the eight blocks of a K-tile of
    256 values reaches only its own block; a batch with split-K and the
    persistent grid."""
    M, N, K = 64, 64, 512
    ops = _int_ops(M, N, K, "mxfp4", 92)
    ops.bsa[5] = np.tile(np.array([125, 126, 128, 129, 127, 129, 125, 126], dtype=np.uint8), K // 256)
    ops.bsb[9] = np.tile(np.array([129, 125, 127, 128, 126, 125, 129, 127], dtype=np.uint8), K // 256)
    C_ref, _ = H.oracle_full(ops)
    for tile in [-1] + FP4_TILES:
        C = H.run(ops, out="f32", tile=tile)
        assert np.array_equal(C, C_ref), tile
    M, N, K, batch = 300, 260, 768, 3
    ops = inputs.make_operands(M, N, K, "mxfp4", "normal", 93, 94, batch=batch)
    refs = [H.oracle_full(ops, bi) for bi in range(batch)]
    for knobs in (dict(), dict(split_k=2), dict(persistent=1), dict(workspace="caller", split_k=3)):
        H.say("mxfp4 batch", knobs)
        C = H.run(ops, out="f32", **knobs)
        for bi in range(batch):
            H.check(C[bi], refs[bi][0], refs[bi][1], "mxfp4", "batch %d %s" % (bi, knobs))


@pytest.mark.parametrize("fmt", ["mxfp6e2m3", "mxfp6e3m2"])
@pytest.mark.parametrize("shape", [(300, 520, 256), (257, 129, 384), (70, 90, 128), (1, 1, 128)])
def test_mxfp6_ragged_full(fmt, shape):
    M, N, K = shape
    ops = inputs.make_operands(M, N, K, fmt, "normal", 850 + M + K, 851 + N)
    C_ref, W = H.oracle_full(ops)
    for tile in [-1] + FP6_TILES:
        for out in ("f32", "bf16"):
            H.say(fmt, "tile", tile, shape, out)
            C = H.run(ops, out=out, tile=tile)
            if out == "f32":
                H.check(C, C_ref, W, fmt, "%s tile %d %s" % (fmt, tile, shape))
            else:
                assert _bf16_ok(C, C_ref, W, fmt), (fmt, tile, shape)


def test_mxfp6_batch_split_and_4096_full():
    M, N, K, batch = 300, 260, 640, 3
    ops = inputs.make_operands(M, N, K, "mxfp6e3m2", "normal", 95, 96, batch=batch)
    refs = [H.oracle_full(ops, bi) for bi in range(batch)]
    for knobs in (dict(), dict(split_k=2), dict(persistent=1), dict(workspace="caller", split_k=3)):
        H.say("mxfp6 batch", knobs)
        C = H.run(ops, out="f32", **knobs)
        for bi in range(batch):
            H.check(C[bi], refs[bi][0], refs[bi][1], "mxfp6e3m2", "batch %d %s" % (bi, knobs))
    M = N = K = 4096
    ops = inputs.make_operands(M, N, K, "mxfp6e2m3", "normal", 103, 104)
    H.say("mxfp6 4096^3")
    C = H.run(ops, out="f32")
    C_ref, W = H.oracle_full(ops)
    H.check(C, C_ref, W, "mxfp6e2m3", "mxfp6 4096^3")


def test_mxfp4_4096_full():
    M = N = K = 4096
    ops = inputs.make_operands(M, N, K, "mxfp4", "normal", 101, 102)
    H.say("mxfp4 4096^3")
    C = H.run(ops, out="f32")
    C_ref, W = H.oracle_full(ops)
    H.check(C, C_ref, W, "mxfp4", "mxfp4 4096^3")


def test_mx_4096_full():
    M = N = K = 4096
    ops = inputs.make_operands(M, N, K, "mxe4m3", "normal", 99, 100)
    H.say("mx 4096^3")
    C = H.run(ops, out="f32")
    C_ref, W = H.oracle_full(ops)
    H.check(C, C_ref, W, "mxe4m3", "mx 4096^3")
