"""GPU parity: libgemm355 (called through its C ABI) against the CPU oracle.

Every case is compared element by element on every output, the full-size
workloads too (in the launch configuration the benchmark times, automatic
plan; all 64 products of the batch); only the 4,000,000-long rows are
sampled.  Exact-integer
inputs make every summation order give the same bits, so those cases demand
bit-identical results through every tile, split, schedule, layout and batch
path (a dropped, duplicated or stale tile, K-slice or LDS stage changes bits).
"""
import os

import numpy as np
import pytest
import torch

from dense_tiled_gemm_fp8_amd import gemm355 as g
from dense_tiled_gemm_fp8_amd import inputs
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

# every entry of the library's tile table, by input type
# matrix-product tiles by input class (convolution tiles: tests/test_gpu_conv.py)
_TILES = [(t, g.gemm355_tile_info(t)["dtype_class"]) for t in range(g.gemm355_num_tiles())
          if g.gemm355_tile_info(t)["op"] == 0]
BF16_TILES = [t for t, c in _TILES if c == 0]
E4M3_TILES = [t for t, c in _TILES if c == 1]


def ops_from(M, N, K, fmt, seed, dist="uniform", batch=0):
    return inputs.make_operands(M, N, K, fmt, dist, seed, seed + 1, batch=batch)


def int_ops(M, N, K, fmt, seed, batch=0, lo=-4, hi=4):
    ga, gb = inputs.rng(seed), inputs.rng(seed + 1)
    nb = max(batch, 1)
    A = np.stack([inputs.small_int_codes(ga, (M, K), fmt, lo, hi) for _ in range(nb)])
    B = np.stack([inputs.small_int_codes(gb, (N, K), fmt, lo, hi) for _ in range(nb)])
    if not batch:
        A, B = A[0], B[0]
    sc = [1.0] * nb
    return inputs.Operands(M, N, K, fmt, A, B, list(sc), list(sc), (seed, seed + 1))


def test_device_is_gfx950():
    assert torch.cuda.is_available()
    props = torch.cuda.get_device_properties(0)
    H.say("device", props.name, getattr(props, "gcnArchName", "?"), props.multi_processor_count)
    assert "gfx950" in getattr(props, "gcnArchName", "gfx950")


@pytest.mark.parametrize("tile", list(range(g.gemm355_num_tiles())))
def test_runtime_occupancy_covers_plan(tile):
    info = g.gemm355_tile_info(tile)
    n = g.gemm355_tile_occupancy(tile)
    H.say("tile", tile, info, "runtime occupancy", n)
    assert n >= info["b_max"]


def test_workload_256_cube_full():
    w = inputs.WORKLOADS[0]
    ops = inputs.workload_operands(w)
    H.say("256^3 bf16 -> f32, seeds", ops.seeds, "sha", inputs.sha256(ops.A, ops.B)[:16])
    C_ref, W = H.oracle_full(ops)
    for knobs in (dict(), dict(split_k=1, persistent=0), dict(split_k=4), dict(persistent=1)):
        H.say("  knobs", knobs)
        C = H.run(ops, out="f32", **knobs)
        H.check(C, C_ref, W, "bf16", "256^3 %s" % knobs)


BF16_SHAPES = [(300, 520, 200), (64, 64, 64), (257, 129, 136), (1, 1, 8), (33, 65, 8), (70, 90, 77),
               (513, 260, 1000)]
E4M3_SHAPES = [(300, 520, 256), (64, 64, 128), (257, 129, 144), (1, 1, 16), (70, 90, 77), (513, 260, 1008)]


@pytest.mark.parametrize("tile", BF16_TILES)
@pytest.mark.parametrize("shape", BF16_SHAPES)
def test_bf16_tiles_ragged_full(tile, shape):
    M, N, K = shape
    ops = ops_from(M, N, K, "bf16", 100 + M + N + K)
    C_ref, W = H.oracle_full(ops)
    for knobs in (dict(split_k=1, persistent=0), dict(split_k=3), dict(split_k=1, persistent=1)):
        H.say("bf16 tile", tile, shape, knobs)
        C = H.run(ops, out="f32", tile=tile, **knobs)
        H.check(C, C_ref, W, "bf16", "bf16 tile %d %s %s" % (tile, shape, knobs))


@pytest.mark.parametrize("tile", E4M3_TILES)
@pytest.mark.parametrize("shape", E4M3_SHAPES)
def test_e4m3_tiles_ragged_full(tile, shape):
    M, N, K = shape
    ops = ops_from(M, N, K, "e4m3", 200 + M + N + K, dist="normal")
    C_ref, W = H.oracle_full(ops)
    for knobs in (dict(split_k=1, persistent=0), dict(split_k=3), dict(split_k=1, persistent=1)):
        H.say("e4m3 tile", tile, shape, knobs)
        C = H.run(ops, out="f32", tile=tile, **knobs)
        H.check(C, C_ref, W, "e4m3", "e4m3 tile %d %s %s" % (tile, shape, knobs))


@pytest.mark.parametrize("fmt,tiles", [("bf16", BF16_TILES), ("e4m3", E4M3_TILES)])
def test_exact_integers_every_path(fmt, tiles):
    """Integers in [-4, 4]: sums are exact in fp32 in any order, so every
    tile, split, schedule and batch path must give the oracle's bits."""
    M, N, K, batch = 300, 270, 384, 3
    ops = int_ops(M, N, K, fmt, 7, batch=batch)
    refs = [H.oracle_full(ops, bi, alpha=1.0)[0] for bi in range(batch)]
    for tile in tiles:
        for knobs in (dict(split_k=1, persistent=0), dict(split_k=2, persistent=0),
                      dict(split_k=3, persistent=1), dict(split_k=1, persistent=1),
                      dict(split_k=5, persistent=0)):
            H.say(fmt, "ints tile", tile, knobs)
            C = H.run(ops, out="f32", tile=tile, **knobs)
            for bi in range(batch):
                assert np.array_equal(C[bi], refs[bi]), (tile, knobs, bi)


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_exact_bf16_output(fmt):
    """bf16 output: integer results with |C| <= 256 are representable, so the
    rounded output is exact."""
    M, N, K = 200, 300, 64
    ops = int_ops(M, N, K, fmt, 11, lo=-2, hi=2)
    ref, _ = H.oracle_full(ops, alpha=1.0)
    assert np.abs(ref).max() <= 256
    for knobs in (dict(split_k=1), dict(split_k=2), dict(persistent=1)):
        H.say(fmt, "bf16-out ints", knobs)
        C = H.run(ops, out="bf16", **knobs)
        assert np.array_equal(C, ref), knobs


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_bf16_output_every_tile(fmt):
    """bf16 C from every product tile, exact integers, with an odd N and a
    leading dimension of N or N + 1: the padding column beyond N stays
    untouched."""
    M, N, K = 130, 99, 64
    ops = int_ops(M, N, K, fmt, 23, lo=-2, hi=2)
    ref, _ = H.oracle_full(ops, alpha=1.0)
    assert np.abs(ref).max() <= 256
    A, B = H.dev(ops.A), H.dev(ops.B)
    sa = sb = None
    if fmt != "bf16":
        sa = torch.tensor(ops.scale_a, dtype=torch.float32, device="cuda")
        sb = torch.tensor(ops.scale_b, dtype=torch.float32, device="cuda")
    for ldc in (N, N + 1):
        for t in (BF16_TILES if fmt == "bf16" else E4M3_TILES):
            H.say(fmt, "bf16 C, tile", t, "ldc", ldc)
            C = torch.full((M, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
            args = g.make_args(M, N, K, A=A, B=B, C=C, ldc=ldc, dtype=H.out_dtype(fmt, "bf16"), tile=t,
                               scale_a=sa, scale_b=sb)
            g.gemm355_gemm_ex(args)
            torch.cuda.synchronize()
            got = C.float().cpu().numpy().astype(np.float64)
            assert np.array_equal(got[:, :N], ref), (t, ldc)
            assert np.isnan(got[:, N:]).all(), (t, ldc)


def _bf16_rne(C_ref: np.ndarray) -> np.ndarray:
    """Exact integer results (binary32-exact) rounded to bf16, nearest even,
    by torch's CPU cast, as binary64."""
    return torch.from_numpy(C_ref.astype(np.float32)).to(torch.bfloat16).double().numpy()


def test_bf16_output_rounds_to_nearest_even():
    """bf16 C is the binary32 result rounded to nearest, ties to even.
    Integers in [-4, 4] over K = 384 give |C| up to ~700: every odd integer
    in (256, 512) is halfway between two bf16 values, so the direct epilogue,
    the split-K combine and the split tail of a persistent grid must all
    pick the even neighbour (257 -> 256, 259 -> 260, 261 -> 260)."""
    assert list(_bf16_rne(np.array([257.0, 259.0, 261.0, 263.0, -257.0, 513.0, 515.0]))) == \
        [256.0, 260.0, 260.0, 264.0, -256.0, 512.0, 516.0]
    M, N, K = 200, 300, 384
    for fmt in ("bf16", "e4m3"):
        ops = int_ops(M, N, K, fmt, 47)
        ref, _ = H.oracle_full(ops, alpha=1.0)
        want = _bf16_rne(ref)
        ties = (np.abs(ref) > 256) & (np.abs(ref) < 512) & (np.mod(ref, 2) == 1)
        assert ties.sum() > 1000 and np.abs(ref).max() > 512
        tiles = BF16_TILES if fmt == "bf16" else E4M3_TILES
        # the first tile with a persistent plan whose partial last round is split
        tail = None
        for t in tiles:
            kw = dict(M=M, N=N, K=K, A=0x10000, B=0x100000, C=0x1000000, dtype=H.out_dtype(fmt, "bf16"), tile=t)
            c = H.split_tail_cus(kw)
            if c is not None:
                tail = dict(tile=t, persistent=1, cus=c)
                break
        assert tail is not None
        runs = [dict(tile=t, split_k=1, persistent=0) for t in tiles]
        runs += [dict(split_k=3), dict(split_k=7, persistent=1), tail]
        for kn in runs:
            H.say(fmt, "bf16 C rounding", kn)
            C = H.run(ops, out="bf16", **kn)
            bad = C != want
            assert not bad.any(), (fmt, kn, int(bad.sum()), C[bad][:4], ref[bad][:4])


def test_power_of_two_scales_exact():
    M, N, K = 128, 192, 256
    ops = int_ops(M, N, K, "e4m3", 13)
    ops.scale_a, ops.scale_b = [0.25], [8.0]
    ref, _ = H.oracle_full(ops, alpha=2.0)
    H.say("e4m3 scales 0.25 x 8")
    C = H.run(ops, out="f32")
    assert np.array_equal(C, ref)


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
@pytest.mark.parametrize("K", [136, 137])
def test_all_layouts(fmt, K):
    """Every storage layout (repacked on the device) against the oracle, and
    the transpose identity (A B)^T = B^T A^T through the layout flags.  With
    K = 137 the K-contiguous operand's rows are not whole 16-byte chunks, so
    one repack launch moves one operand by rows and the other by transposed
    blocks."""
    M, N = 150, 98
    ops = ops_from(M, N, K, fmt, 17, dist="normal")
    a_log = ops.A                       # M x K logical
    b_log = np.ascontiguousarray(ops.B.T)  # K x N logical
    C_ref, W = H.oracle_full(ops)
    alpha = H.alpha_of(ops)
    for layout in (g.A_ROW_B_COL, g.A_ROW_B_ROW, g.A_COL_B_COL, g.A_COL_B_ROW):
        a_row = layout in (g.A_ROW_B_COL, g.A_ROW_B_ROW)
        b_col = layout in (g.A_ROW_B_COL, g.A_COL_B_COL)
        A_st = a_log if a_row else np.ascontiguousarray(a_log.T)
        B_st = np.ascontiguousarray(b_log.T) if b_col else b_log
        lda = K if a_row else M
        ldb = K if b_col else N
        H.say(fmt, "layout", layout)
        C = H.run(ops, out="f32", layout=layout, A_dev=H.dev(A_st), B_dev=H.dev(B_st), lda=lda, ldb=ldb)
        H.check(C, C_ref, W, fmt, "layout %d" % layout)
    # transpose identity with exact integers: N x M result from swapped roles
    iops = int_ops(M, N, K, fmt, 19)
    C1 = H.run(iops, out="f32")
    swapped = inputs.Operands(N, M, K, fmt, iops.B, iops.A, [1.0], [1.0])
    C2 = H.run(swapped, out="f32")
    assert np.array_equal(C1, C2.T)


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_rows_in_place_misaligned_with_nan_padding(fmt):
    """K-contiguous rows read in place: the operands start one element past
    a 16-byte boundary, rows are lda = K + 3 and ldb = K + 5 elements apart
    (no row 16-byte aligned), K = 77 ends inside a 16-byte chunk, and every
    element outside the matrices (the row padding and what follows the last
    row) is a NaN code.  The bytes of the last chunk past K must be cleared
    before the product, so exact-integer results are the oracle's bits
    through every tile that reads rows in place, split-K and the persistent
    grid included."""
    M, N, K = 130, 200, 77
    lda, ldb = K + 3, K + 5
    ops = int_ops(M, N, K, fmt, 53)
    nan = np.uint16(0x7FC0) if fmt == "bf16" else np.uint8(0x7F)
    dt = np.uint16 if fmt == "bf16" else np.uint8

    def padded(codes, rows, ld):
        buf = np.full(1 + rows * ld + 64, nan, dtype=dt)
        buf[1:1 + rows * ld].reshape(rows, ld)[:, :K] = codes
        return H.dev(buf)

    Abuf, Bbuf = padded(ops.A, M, lda), padded(ops.B, N, ldb)
    ref, _ = H.oracle_full(ops, alpha=1.0)
    tiles = [t for t in (BF16_TILES if fmt == "bf16" else E4M3_TILES)
             if g.gemm355_plan(g.make_args(M, N, K, A=Abuf[1:], lda=lda, B=Bbuf[1:], ldb=ldb,
                                           C=0x200000000000, dtype=H.out_dtype(fmt, "f32"), tile=t))["repack"] == 0]
    assert len(tiles) >= 5
    for tile in [-1] + tiles:
        for knobs in (dict(split_k=1, persistent=0), dict(split_k=3), dict(persistent=1)):
            H.say(fmt, "in place, NaN padding, tile", tile, knobs)
            C = H.run(ops, out="f32", tile=tile, A_dev=Abuf[1:], B_dev=Bbuf[1:], lda=lda, ldb=ldb, **knobs)
            assert np.array_equal(C, ref), (fmt, tile, knobs)


@pytest.mark.parametrize("fmt,M,N,K", [("bf16", 2600, 2500, 2001), ("e4m3", 3200, 3200, 3201)])
def test_rows_misaligned_repacked_large(fmt, M, N, K):
    """Rows that are not 16-byte aligned in a product large enough for the
    planner to repack them (dense-MFMA time at peak of 10 us or more): the
    operands start one element past a 16-byte boundary, rows are K + 3 and
    K + 5 elements apart, K ends inside a 16-byte chunk and every element
    outside the matrices is a NaN code.  The repack pass must copy exactly
    the K elements of each row and zero the rest of its padded row, so
    exact-integer results are the oracle's bits."""
    lda, ldb = K + 3, K + 5
    ops = int_ops(M, N, K, fmt, 57, lo=-1, hi=1)
    nan = np.uint16(0x7FC0) if fmt == "bf16" else np.uint8(0x7F)
    dt = np.uint16 if fmt == "bf16" else np.uint8

    def padded(codes, rows, ld):
        buf = np.full(1 + rows * ld + 64, nan, dtype=dt)
        buf[1:1 + rows * ld].reshape(rows, ld)[:, :K] = codes
        return H.dev(buf)

    Abuf, Bbuf = padded(ops.A, M, lda), padded(ops.B, N, ldb)
    p = g.gemm355_plan(g.make_args(M, N, K, A=Abuf[1:], lda=lda, B=Bbuf[1:], ldb=ldb, C=0x200000000000,
                                   dtype=H.out_dtype(fmt, "f32")))
    H.say(fmt, M, N, K, "misaligned rows: repack", p["repack"], "tile", p["tile"])
    assert p["repack"] == 3
    ref, _ = H.oracle_full(ops, alpha=1.0)
    C = H.run(ops, out="f32", A_dev=Abuf[1:], B_dev=Bbuf[1:], lda=lda, ldb=ldb)
    assert np.array_equal(C, ref)


@pytest.mark.parametrize("fmt,K", [("bf16", 5), ("bf16", 13), ("bf16", 77), ("e4m3", 7), ("e4m3", 29),
                                   ("e4m3", 141)])
def test_row_repack_edges(fmt, K):
    """The row repack pass on its edge cases: a tile whose copy schedule
    does not clear K tails is forced, so rows that end inside a 16-byte
    chunk are repacked; the rows start one element past a 16-byte boundary
    and lie K + 3 / K + 5 elements apart with NaN codes in between.  K
    covers rows shorter than one chunk (read byte by byte), rows of one
    whole chunk and a partial one, and longer rows; every output is the
    oracle's exact sum."""
    M, N = 130, 200
    lda, ldb = K + 3, K + 5
    ops = int_ops(M, N, K, fmt, 59)
    nan = np.uint16(0x7FC0) if fmt == "bf16" else np.uint8(0x7F)
    dt = np.uint16 if fmt == "bf16" else np.uint8

    def padded(codes, rows, ld):
        buf = np.full(1 + rows * ld + 64, nan, dtype=dt)
        buf[1:1 + rows * ld].reshape(rows, ld)[:, :K] = codes
        return H.dev(buf)

    Abuf, Bbuf = padded(ops.A, M, lda), padded(ops.B, N, ldb)
    cls = 0 if fmt == "bf16" else 1
    tile = [t for t in range(g.gemm355_num_tiles()) if g.gemm355_tile_info(t)["dtype_class"] == cls
            and g.gemm355_tile_info(t)["op"] == 0
            and g.gemm355_plan(g.make_args(M, N, K, A=Abuf[1:], lda=lda, B=Bbuf[1:], ldb=ldb, C=0x200000000000,
                                           dtype=H.out_dtype(fmt, "f32"), tile=t))["repack"] == 3][0]
    H.say(fmt, "K", K, "row repack through forced tile", tile)
    ref, _ = H.oracle_full(ops, alpha=1.0)
    C = H.run(ops, out="f32", tile=tile, A_dev=Abuf[1:], B_dev=Bbuf[1:], lda=lda, ldb=ldb)
    assert np.array_equal(C, ref)


def test_persistent_on_off_bit_identical():
    """Same tile and the same uniform split: the persistent loop only changes
    which workgroup runs a unit, so results are bit-identical."""
    M, N, K = 1100, 700, 1500
    ops = ops_from(M, N, K, "bf16", 23, dist="normal")
    for tile, s in ((0, 1), (1, 2), (2, 3)):
        H.say("persistent on/off tile", tile, "split", s)
        C0 = H.run(ops, out="f32", tile=tile, split_k=s, persistent=0)
        C1 = H.run(ops, out="f32", tile=tile, split_k=s, persistent=1 if s > 1 else 0)
        assert np.array_equal(C0, C1)
    C_ref, W = H.oracle_full(ops)
    H.check(C0, C_ref, W, "bf16", "persistent")


def test_split_invariant_float():
    M, N, K = 256, 192, 8192
    ops = ops_from(M, N, K, "bf16", 29, dist="normal_sqrtk")
    C_ref, W = H.oracle_full(ops)
    base = H.run(ops, out="f32", split_k=1, persistent=0)
    H.check(base, C_ref, W, "bf16", "split 1")
    for s in (2, 7, 32, 128):
        H.say("split", s)
        C = H.run(ops, out="f32", split_k=s)
        H.check(C, C_ref, W, "bf16", "split %d" % s)
        assert np.all(np.abs(C - base) <= 2e-3 * W + 2e-6)


def test_leading_dims_offsets_and_workspace():
    M, N, K = 200, 136, 96
    ops = ops_from(M, N, K, "bf16", 31)
    C_ref, W = H.oracle_full(ops)
    # padded leading dimensions (16-byte aligned rows: main loop reads directly)
    Aw = np.zeros((M, K + 24), dtype=np.uint16)
    Aw[:, :K] = ops.A
    Bw = np.zeros((N, K + 40), dtype=np.uint16)
    Bw[:, :K] = ops.B
    H.say("ld padded")
    C = H.run(ops, out="f32", A_dev=H.dev(Aw), B_dev=H.dev(Bw), lda=K + 24, ldb=K + 40)
    H.check(C, C_ref, W, "bf16", "padded ld")
    # an A that starts one element past a 16-byte boundary (repack path)
    buf = H.dev(np.concatenate([np.zeros(1, np.uint16), ops.A.reshape(-1)]))
    H.say("misaligned A")
    C = H.run(ops, out="f32", A_dev=buf[1:])
    H.check(C, C_ref, W, "bf16", "misaligned A")
    # output with ldc > N
    Cbig = torch.full((M, N + 8), 7.0, dtype=torch.float32, device="cuda")
    args = g.make_args(M, N, K, A=H.dev(ops.A), B=H.dev(ops.B), C=Cbig, ldc=N + 8)
    H.say("ldc padded")
    g.gemm355_gemm_ex(args)
    torch.cuda.synchronize()
    out = Cbig.cpu().numpy().astype(np.float64)
    H.check(out[:, :N], C_ref, W, "bf16", "ldc")
    assert np.all(out[:, N:] == 7.0)
    # caller workspace and library scratch give the same bits
    for knobs in (dict(split_k=4), dict(persistent=1, tile=1)):
        H.say("workspace", knobs)
        C1 = H.run(ops, out="f32", workspace="caller", **knobs)
        C2 = H.run(ops, out="f32", **knobs)
        assert np.array_equal(C1, C2)


def test_library_scratch_concurrent_calls_one_stream():
    """Host threads calling split-K products on ONE stream with library-owned
    scratch, each growing the buffer in turn: every call's kernels are
    enqueued as a group (no call's main pass overwrites partial sums another
    call's combine pass still needs, no buffer is freed under a call), so
    every result is the oracle's, bit for bit (exact integers)."""
    import threading
    stream = torch.cuda.current_stream()
    jobs = []
    for t in range(6):
        M, N, K = 96 + 32 * t, 80 + 16 * t, 1024 * (t + 1)
        ops = int_ops(M, N, K, "bf16", 300 + t)
        ref, _ = H.oracle_full(ops, alpha=1.0)
        A, B = H.dev(ops.A), H.dev(ops.B)
        Cs = [torch.full((M, N), float("nan"), device="cuda") for _ in range(8)]
        jobs.append((M, N, K, A, B, Cs, ref))
    torch.cuda.synchronize()
    errors = []

    def worker(job, split):
        M, N, K, A, B, Cs, _ = job
        try:
            for i, C in enumerate(Cs):
                a = g.make_args(M, N, K, A=A, B=B, C=C, dtype=g.BF16_F32, split_k=split + (i % 3),
                                tile=2)
                g.gemm355_gemm_ex(a, stream)
        except Exception as e:   # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j, 4 + 2 * t)) for t, j in enumerate(jobs)]
    H.say("scratch: %d threads x 8 split-K calls on one stream" % len(threads))
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (M, N, K, A, B, Cs, ref) in jobs:
        for C in Cs:
            assert np.array_equal(C.double().cpu().numpy(), ref), (M, N, K)


def test_library_scratch_cap_enomem():
    """Library-owned scratch over the cap of gemm355_set_scratch_limit: the
    call returns ENOMEM before launching anything (C keeps its NaN fill) and
    a repacking call is refused the same way; at a cap equal to the plan's
    need the same split-K call runs and gives the oracle's bits."""
    M, N, K = 200, 168, 4096
    ops = int_ops(M, N, K, "bf16", 77)
    ref, _ = H.oracle_full(ops, alpha=1.0)
    A, B = H.dev(ops.A), H.dev(ops.B)
    C = torch.full((M, N), float("nan"), device="cuda")
    a = g.make_args(M, N, K, A=A, B=B, C=C, dtype=g.BF16_F32, split_k=4, tile=2)
    need = g.gemm355_plan(a)["workspace_bytes"]
    assert need > 0
    prev = g.gemm355_set_scratch_limit(need - 1)
    try:
        H.say("scratch cap", need - 1, "below the need", need)
        with pytest.raises(g.Gemm355Error) as e:
            g.gemm355_gemm_ex(a)
        assert e.value.status == g.ENOMEM
        # a caller workspace is not subject to the cap
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        Cw = torch.full((M, N), float("nan"), device="cuda")
        g.gemm355_gemm_ex(g.make_args(M, N, K, A=A, B=B, C=Cw, dtype=g.BF16_F32, split_k=4, tile=2,
                                      workspace=ws, workspace_bytes=need))
        # a cap of 0 refuses every call that needs scratch, not the others
        assert g.gemm355_set_scratch_limit(0) == need - 1
        with pytest.raises(g.Gemm355Error) as e:
            g.gemm355_gemm_ex(a)
        assert e.value.status == g.ENOMEM
        C0 = torch.full((M, N), float("nan"), device="cuda")
        g.gemm355_gemm_ex(g.make_args(M, N, K, A=A, B=B, C=C0, dtype=g.BF16_F32, split_k=1, persistent=0,
                                      tile=2))
        torch.cuda.synchronize()
        assert torch.isnan(C).all()
        g.gemm355_set_scratch_limit(need)
        H.say("scratch cap", need)
        g.gemm355_gemm_ex(a)
        torch.cuda.synchronize()
    finally:
        g.gemm355_set_scratch_limit(prev)
    for out in (C, Cw, C0):
        assert np.array_equal(out.double().cpu().numpy(), ref)


def test_binding_imported_before_torch():
    """A fresh process that imports the binding before anything else: the
    binding loads PyTorch first, so the library binds to torch's HIP runtime
    (a second runtime loaded from the system ROCm would make torch's device
    memory foreign to the library's launches) and a product is exact."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from dense_tiled_gemm_fp8_amd import gemm355 as g\n"
        "from tests import gpu_helpers as H\n"
        "maps = open('/proc/self/maps').read()\n"
        "libs = set(l.split()[-1] for l in maps.split('\\n') if 'libamdhip64' in l)\n"
        "assert len(libs) == 1, libs\n"
        "ops = H.exact_ops(300, 200, 256, 'bf16', 123)\n"
        "ref, _ = H.oracle_full(ops, 0, alpha=1.0)\n"
        "C = H.run(ops, out='f32')\n"
        "assert (C == ref).all()\n"
        "print('one runtime, exact')\n") % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    H.say("binding imported first, fresh process")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "one runtime, exact" in r.stdout, r.stdout + r.stderr


def test_degenerate_sizes():
    ops = ops_from(5, 7, 0, "bf16", 37)
    H.say("K = 0")
    C = H.run(ops, out="f32", A_dev=H.dev(np.zeros(8, np.uint16)), B_dev=H.dev(np.zeros(8, np.uint16)))
    assert np.all(C == 0.0)
    H.say("M = 0")
    Cz = torch.full((1, 4), 3.0, device="cuda")
    g.gemm355_gemm(0, 4, 16, H.dev(np.zeros(64, np.uint16)), 16, H.dev(np.zeros(64, np.uint16)), 16,
                   Cz, 4, g.BF16_F32)
    torch.cuda.synchronize()
    assert torch.all(Cz == 3.0)
    H.say("1x1x1")
    one = ops_from(1, 1, 1, "bf16", 41)
    C_ref, W = H.oracle_full(one)
    C = H.run(one, out="f32")
    H.check(C, C_ref, W, "bf16", "1x1x1")
    H.say("gemm355_gemm entry point")
    ops = ops_from(130, 70, 48, "bf16", 43)
    C_ref, W = H.oracle_full(ops)
    Cg = torch.full((130, 70), float("nan"), device="cuda")
    g.gemm355_gemm(130, 70, 48, H.dev(ops.A), 48, H.dev(ops.B), 48, Cg, 70, g.BF16_F32)
    torch.cuda.synchronize()
    H.check(Cg.cpu().numpy().astype(np.float64), C_ref, W, "bf16", "gemm355_gemm")


def test_largest_row_offsets_sampled():
    """K = 4,000,000 bf16 (8 MB rows): a tile's 256 rows span just under the
    2^31 bytes of 32-bit buffer offsets the main loop uses, and the split-K
    slices reach the far end of every row.  Sampled outputs (corners and
    ragged edges included) against the oracle."""
    M, N, K = 300, 200, 4_000_000
    r = np.random.Generator(np.random.PCG64(1234))
    lut = inputs.to_bf16_codes(np.arange(-4, 5, dtype=np.float64))
    A = lut[r.integers(0, 9, size=(M, K), dtype=np.uint8)]
    B = lut[r.integers(0, 9, size=(N, K), dtype=np.uint8)]
    ops = inputs.Operands(M, N, K, "bf16", A, B, [1.0], [1.0], (1234, 1234))
    a = g.make_args(M, N, K, A=0x10000, B=0x1000000000, C=0x200000000000, cus=256)
    p = g.gemm355_plan(a)
    assert 256 * K * 2 <= 0x7FFF0000
    H.say("K = 4e6, plan", p["T_M"], p["T_N"], "split", p["split"], "tail", p["tail_tiles"], p["tail_split"])
    C = H.run(ops, out="f32")
    rows, cols = H.sample_positions(M, N, 40, 3)
    c, w = H.oracle_entries(ops, rows, cols)
    H.check(C[rows, cols], c, w, "bf16", "K = 4e6")


# ------------------------------------------------------------ full-size workloads
#
# The five workloads at their full sizes, in the launch configuration the
# benchmark times (automatic plan), compared with the oracle on EVERY output
# (all 64 products of the batch) at the stated tolerances.  The oracle takes
# a few seconds per 10^11 multiply-adds on the host's cores.

def _full(ops, out, what=""):
    H.say(what, "sha", inputs.sha256(ops.A, ops.B)[:16])
    A_dev, B_dev = H.dev(ops.A), H.dev(ops.B)
    C = H.run(ops, out=out, A_dev=A_dev, B_dev=B_dev)
    del A_dev, B_dev
    Cb = C if ops.batch > 1 else C[None]
    assert np.all(np.isfinite(Cb))
    for bi in range(ops.batch):
        C_ref, W = H.oracle_full(ops, bi)
        H.check(Cb[bi], C_ref, W, ops.fmt, "%s entry %d" % (what, bi))
    H.say(what, "all", Cb.size, "outputs within tolerance")
    return C


def test_workload_4096_cube_bf16_out():
    w = inputs.WORKLOADS[1]
    ops = inputs.workload_operands(w)
    _full(ops, "bf16", what="4096^3 bf16->bf16")


@pytest.mark.parametrize("si", [0, 1, 2])
def test_workload_ragged(si):
    w = inputs.WORKLOADS[2]
    ops = inputs.workload_operands(w, si)
    _full(ops, "f32", what="ragged %s" % (w.shapes[si],))


@pytest.mark.parametrize("si", [0, 1, 2])
def test_workload_split_k(si):
    w = inputs.WORKLOADS[3]
    ops = inputs.workload_operands(w, si)
    _full(ops, "f32", what="split-K %s" % (w.shapes[si],))


def test_workload_e4m3_8192_cube():
    w = inputs.WORKLOADS[4]
    ops = inputs.workload_operands(w)
    _full(ops, "f32", what="e4m3 8192^3")


def test_workload_e4m3_batch64():
    w = inputs.WORKLOADS[5]
    ops = inputs.workload_operands(w)
    assert ops.batch == 64 and len(set(ops.scale_a)) > 1
    _full(ops, "f32", what="e4m3 batch 64x(512,1024,4096)")


def test_unit_stamps_cover_every_unit():
    """The per-unit clock hook: every unit of a persistent split schedule
    records start <= loop end <= stores issued <= end, the product is
    unchanged by recording, and the busy fraction the stamps give lies in
    (0, 1]."""
    M, N, K = 1500, 1300, 2048
    ops = ops_from(M, N, K, "bf16", 37, dist="normal")
    A, B = H.dev(ops.A), H.dev(ops.B)
    C0 = H.empty_c(1, M, N, "f32")
    C1 = H.empty_c(1, M, N, "f32")
    for tile, split, pers in ((1, 3, 1), (0, 1, 0), (2, 1, 1)):
        args = g.make_args(M, N, K, A=A, B=B, C=C0, dtype=g.BF16_F32, tile=tile, split_k=split,
                           persistent=pers)
        p = g.gemm355_plan(args)
        H.say("stamps tile", tile, "split", split, "persistent", pers, "units", p["units"], "grid", p["grid"])
        g.gemm355_gemm_ex(args)
        stamps = torch.zeros(6 * p["units"], dtype=torch.int64, device="cuda")
        args2 = g.make_args(M, N, K, A=A, B=B, C=C1, dtype=g.BF16_F32, tile=tile, split_k=split,
                            persistent=pers, unit_stamps=stamps)
        g.gemm355_gemm_ex(args2)
        torch.cuda.synchronize()
        assert torch.equal(C0, C1)
        st = stamps.view(-1, 6).cpu().numpy()
        assert (st[:, 0] > 0).all() and (st[:, 1] >= st[:, 0]).all()
        assert (st[:, 3] > st[:, 2]).all()
        # start <= main loop done <= stores issued <= stores complete (shader clock)
        assert (st[:, 4] >= st[:, 2]).all() and (st[:, 5] >= st[:, 4]).all() and (st[:, 3] >= st[:, 5]).all()
        # shader cycles per real-time tick (100 MHz): a clock between 0.3 and 3 GHz
        mhz = 100.0 * float((st[:, 3] - st[:, 2]).sum()) / max(float((st[:, 1] - st[:, 0]).sum()), 1.0)
        H.say("  shader clock from the stamps (MHz)", mhz)
        assert 300.0 < mhz < 3000.0
        busy = float((st[:, 1] - st[:, 0]).sum())
        span = float(st[:, 1].max() - st[:, 0].min())
        eta = busy / (p["S"] * p["b"] * span)
        H.say("  measured busy fraction", eta)
        assert 0.0 < eta <= 1.0
    C_ref, W = H.oracle_full(ops)
    H.check(C1.float().cpu().numpy().astype(np.float64), C_ref, W, "bf16", "stamps")
