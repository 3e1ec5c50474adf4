"""Host-side checks of libgemm355 through its C ABI (no kernel launches).

* every symbol include/gemm355.h declares is exported;
* the wave- and padding-efficiency queries equal the exact rationals of the
  bookkeeping oracle bit for bit;
* K-slices, tile grid, padded sizes, resident workgroups and schedule
  efficiency of the plans equal the oracle's;
* the work units a plan hands to the kernels cover every (tile, K-tile) once;
* argument errors are reported before anything is launched.
"""
import math
import os
import random
import re
import struct
from fractions import Fraction

import pytest

from oracle import bookkeeping as bk
from oracle import conv as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def g():
    from dense_tiled_gemm_fp8_amd import gemm355
    return gemm355


def bits(x: float) -> bytes:
    return struct.pack("<d", x)


def test_header_symbols_exported(g):
    hdr = open(os.path.join(ROOT, "include", "gemm355.h")).read()
    declared = set(re.findall(r"GEMM355_API\s+[\w\s\*]+?\b(gemm355_\w+)\s*\(", hdr))
    assert declared, "no declarations found"
    assert declared == set(g.EXPORTED)
    for name in declared:
        assert hasattr(g._lib, name), name


def test_binding_holds_no_method_arithmetic():
    """The Python binding only marshals arguments: no function in it does
    arithmetic (sizes, offsets, output extents all come from the library).
    The only binary operators allowed are %-formatting of message strings."""
    import ast
    path = os.path.join(ROOT, "dense_tiled_gemm_fp8_amd", "gemm355.py")
    tree = ast.parse(open(path).read())
    bad = []
    for fn in [n for n in ast.walk(tree) if isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef))]:
        for node in [n for stmt in fn.body for n in ast.walk(stmt)]:
            if isinstance(node, ast.AugAssign):
                bad.append((fn.name, node.lineno))
            elif isinstance(node, ast.BinOp):
                if isinstance(node.op, ast.Mod) and isinstance(node.left, ast.Constant) and \
                        isinstance(node.left.value, str):
                    continue
                bad.append((fn.name, node.lineno))
            elif isinstance(node, ast.UnaryOp) and isinstance(node.op, (ast.USub, ast.Invert)):
                bad.append((fn.name, node.lineno))
    assert not bad, "arithmetic in the binding: %s" % bad


def test_noalloc_host_checks(g):
    """gemm355_gemm_noalloc refuses a caller workspace (EINVAL) and a plan
    whose scratch exceeds its fixed 64 MiB array (ETOOBIG) before any device
    work."""
    base = dict(A=0x10000, B=0x1000000000, C=0x200000000000, cus=256)
    big = g.make_args(4096, 4096, 4096, split_k=8, tile=0, **base)
    assert g.gemm355_plan(big)["workspace_bytes"] == 256 * 8 * 256 * 256 * 4
    with pytest.raises(g.Gemm355Error) as e:
        g.gemm355_gemm_noalloc(big, stream=0)
    assert e.value.status == g.ETOOBIG
    with pytest.raises(g.Gemm355Error) as e:
        g.gemm355_gemm_noalloc(g.make_args(64, 64, 64, workspace=0x300000000000, workspace_bytes=1 << 20,
                                           **base), stream=0)
    assert e.value.status == g.EINVAL
    assert "fixed buffer" in g.gemm355_status_string(g.ETOOBIG)


def test_eta_wave_bit_exact(g):
    rnd = random.Random(0)
    cases = [(24, 148, 1), (12, 148, 1), (256, 256, 1), (272, 256, 1), (1, 256, 1), (752, 256, 4)]
    cases += [(rnd.randint(1, 10 ** 7), rnd.randint(1, 512), rnd.randint(1, 8)) for _ in range(3000)]
    for G, S, b in cases:
        assert bits(g.gemm355_eta_wave(G, S, b)) == bits(float(bk.eta_wave(G, S, b))), (G, S, b)


def test_eta_pad_bit_exact(g):
    rnd = random.Random(1)
    cases = [(4096, 4096, 4096, 256, 256, 64), (4000, 4000, 4000, 256, 256, 64),
             (4097, 4095, 4104, 256, 256, 64), (1000, 3000, 777, 64, 64, 64)]
    cases += [(rnd.randint(1, 1 << 20), rnd.randint(1, 1 << 20), rnd.randint(1, 1 << 20),
               rnd.choice([16, 32, 64, 128, 256]), rnd.choice([16, 64, 256]),
               rnd.choice([32, 64, 128])) for _ in range(3000)]
    for c in cases:
        assert bits(g.gemm355_eta_pad(*c)) == bits(float(bk.eta_pad(*c))), c


def test_eta_queries_reject_invalid(g):
    import math
    assert math.isnan(g.gemm355_eta_wave(0, 256, 1))
    assert math.isnan(g.gemm355_eta_wave(5, 0, 1))
    assert math.isnan(g.gemm355_eta_pad(0, 1, 1, 1, 1, 1))
    assert math.isnan(g.gemm355_eta_pad(1, 1, 1, 1, 0, 1))


def test_kslice_matches_oracle(g):
    rnd = random.Random(2)
    for _ in range(2000):
        nK = rnd.randint(0, 1 << 22)
        s = rnd.randint(1, 256)
        i = rnd.randrange(s)
        assert g.gemm355_kslice(nK, s, i) == bk.kslice(nK, s, i)
    with pytest.raises(g.Gemm355Error):
        g.gemm355_kslice(10, 0, 0)
    with pytest.raises(g.Gemm355Error):
        g.gemm355_kslice(10, 4, 4)


# shapes: the named workloads plus ragged and degenerate ones
PLAN_SHAPES = [
    (256, 256, 256, 1, 0), (4096, 4096, 4096, 1, 1), (4000, 4000, 4000, 1, 0),
    (4097, 4095, 4104, 1, 0), (1000, 3000, 777, 1, 0), (256, 256, 65536, 1, 0),
    (128, 512, 131072, 1, 0), (64, 64, 262144, 1, 0), (8192, 8192, 8192, 1, 2),
    (512, 1024, 4096, 64, 2), (1, 1, 1, 1, 0), (17, 300, 40, 3, 2), (5000, 33, 9000, 1, 0),
    (1000, 900, 700, 1, 3), (64, 4096, 8192, 2, 4), (8192, 8192, 8192, 1, 5),
    (512, 1024, 4096, 64, 5), (1000, 900, 768, 1, 5), (100, 70, 131072, 1, 5),
    (8192, 8192, 8192, 1, 6), (300, 500, 512, 3, 6), (4096, 4096, 4096, 1, 7), (300, 520, 384, 2, 7),
]
PLAN_DTYPES = ["BF16_F32", "BF16_BF16", "E4M3_F32", "E5M2_F32", "E4M3_E5M2_BF16", "MXE4M3_F32", "MXFP4_F32",
               "MXFP6_E3M2_BF16"]

KNOBS = [dict(), dict(split_k=1, persistent=0), dict(split_k=3), dict(split_k=1, persistent=1),
         dict(split_k=5, persistent=1), dict(tile=1), dict(tile=2, persistent=1, split_k=1)]


def _plan_and_check(g, M, N, K, batch, dtype, knobs, exact_tile=False):
    if exact_tile:
        pass
    elif "tile" in knobs and dtype in (g.E4M3_F32, g.E5M2_F32, g.E4M3_E5M2_BF16):
        knobs = dict(knobs, tile=knobs["tile"] + 3)
    elif "tile" in knobs and dtype == g.MXE4M3_F32:
        knobs = dict(knobs, tile=knobs["tile"] + 48)           # the block-scaled 128x128 tiles
    elif "tile" in knobs and dtype == g.MXFP4_F32:
        knobs = dict(knobs, tile=knobs["tile"] + 51)           # the FP4 128x128 tiles
    elif "tile" in knobs and dtype == g.MXFP6_E3M2_BF16:
        knobs = dict(knobs, tile=knobs["tile"] + 59)           # the FP6 128x128 tiles
    if dtype in (g.MXE4M3_F32, g.MXFP4_F32, g.MXFP6_E3M2_BF16):
        knobs = dict(knobs, block_scale_a=0x300000000000, block_scale_b=0x380000000000)
    a = g.make_args(M, N, K, A=0x10000, B=0x1000000000, C=0x200000000000, dtype=dtype,
                    batch=batch, stride_a=M * K, stride_b=N * K, stride_c=M * N, cus=256, **knobs)
    p = g.gemm355_plan(a)
    info = g.gemm355_tile_info(p["tile"])
    S, b = 256, p["b"]
    assert p["S"] == S
    # tile grid, padding, K-tiles (equations for G and the padded dimensions)
    tm, tn = bk.ceil_div(M, p["T_M"]), bk.ceil_div(N, p["T_N"])
    assert p["G"] == batch * bk.tile_grid(M, N, p["T_M"], p["T_N"])
    assert p["nK"] == bk.ceil_div(K, p["T_K"])
    assert (p["M_pad"], p["N_pad"], p["K_pad"]) == (bk.padded(M, p["T_M"]), bk.padded(N, p["T_N"]),
                                                    bk.padded(K, p["T_K"]))
    assert Fraction(p["eta_wave_num"], p["eta_wave_den"]) == bk.eta_wave(p["G"], S, b)
    assert Fraction(p["eta_pad_num"], p["eta_pad_den"]) == bk.eta_pad(M, N, K, p["T_M"], p["T_N"], p["T_K"])
    # resident workgroups: the launched b never exceeds the oracle's bound
    # gfx950 unit: 160 KiB LDS, 4 SIMDs x 64 lanes x 512 registers, granule
    # 8, at most 8 waves per SIMD
    bmax = bk.resident_per_sm(info["lds_bytes"], 160 * 1024, p["vgpr_budget"], 8,
                              64 * info["waves"], 4 * 64 * 512, max_ctas=32 // info["waves"])["b"]
    assert info["b_max"] == bmax
    assert 1 <= b <= bmax
    # schedule: rebuild the unit list from the oracle's policy
    if p["split"] > 1:
        units = bk.schedule_units(p["G"], p["nK"], s=p["split"])
    elif p["tail_tiles"]:
        units = bk.schedule_units(p["G"], p["nK"], tail_split=True, P=S * b)
        assert bk.tail_split_factor(p["G"], p["nK"], S * b) == p["tail_split"]
    else:
        units = bk.schedule_units(p["G"], p["nK"])
    assert len(units) == p["units"]
    assert Fraction(p["eta_sched_num"], p["eta_sched_den"]) == bk.eta_sched_units(units, S, b, grid=p["grid"])
    if p["persistent"]:
        assert p["grid"] == min(p["units"], S * b)
    else:
        assert p["grid"] == p["units"]
    return a, p


@pytest.mark.parametrize("M,N,K,batch,dt", PLAN_SHAPES)
def test_plan_bookkeeping(g, M, N, K, batch, dt):
    dtype = getattr(g, PLAN_DTYPES[dt])
    for knobs in KNOBS:
        _plan_and_check(g, M, N, K, batch, dtype, knobs)


@pytest.mark.parametrize("M,N,K,batch,dt", [s for s in PLAN_SHAPES if s[0] * s[1] * s[3] <= 5000 * 5000])
def test_units_cover_every_k_tile_once(g, M, N, K, batch, dt):
    dtype = getattr(g, PLAN_DTYPES[dt])
    for knobs in KNOBS:
        a, p = _plan_and_check(g, M, N, K, batch, dtype, knobs)
        if p["units"] > 20000:
            continue
        tm, tn = bk.ceil_div(M, p["T_M"]), bk.ceil_div(N, p["T_N"])
        seen = {}
        for u in range(p["units"]):
            bt, i, j, kb, ke = g.gemm355_unit(a, u)
            assert 0 <= bt < batch and 0 <= i < tm and 0 <= j < tn and 0 <= kb < ke <= p["nK"]
            key = (bt, i, j)
            seen.setdefault(key, []).append((kb, ke))
        assert len(seen) == p["G"]
        for ranges in seen.values():
            ranges.sort()
            assert ranges[0][0] == 0 and ranges[-1][1] == p["nK"]
            for (b0, e0), (b1, e1) in zip(ranges, ranges[1:]):
                assert e0 == b1
            if p["split"] > 1:
                assert ranges == bk.kslices(p["nK"], p["split"])
        with pytest.raises(g.Gemm355Error):
            g.gemm355_unit(a, p["units"])


def test_plan_bookkeeping_random(g):
    """Seeded random shapes (log-uniform M, N up to 9000 and K up to 300000,
    batches up to 7), every input dtype class, the knob sets and (in about a
    third of the cases) a forced tile of the matching class: each plan
    satisfies the oracle's grid, padding, eta, residency and schedule
    arithmetic, and where the unit list is short every tile's K-tiles are
    covered exactly once.  Block-scaled K is a multiple of 128, FP4's of 256
    (the planner refuses any other)."""
    rnd = random.Random(7)
    classes = {"BF16": 0, "E4M3": 1, "E5M2": 1, "MXE4M3": 2, "MXFP4": 3, "MXFP6": 4}
    by_class = {}
    for t in range(g.gemm355_num_tiles()):
        info = g.gemm355_tile_info(t)
        if info["op"] == 0:
            by_class.setdefault(info["dtype_class"], []).append(t)
    for _ in range(1500):
        M = int(math.exp(rnd.uniform(0, math.log(9000))))
        N = int(math.exp(rnd.uniform(0, math.log(9000))))
        K = int(math.exp(rnd.uniform(0, math.log(300000))))
        batch = rnd.choice([1, 1, 1, 2, 3, 7])
        name = rnd.choice(PLAN_DTYPES)
        dtype = getattr(g, name)
        if name.startswith("MX"):
            step = 256 if name.startswith("MXFP4") else 128
            K = -(-K // step) * step
        knobs = rnd.choice(KNOBS)
        exact = rnd.random() < 0.3
        if exact:
            cls = classes[name.split("_")[0]]
            knobs = dict(rnd.choice(KNOBS[:5]), tile=rnd.choice(by_class[cls]))
        a, p = _plan_and_check(g, M, N, K, batch, dtype, knobs, exact_tile=exact)
        if exact:
            assert p["tile"] == knobs["tile"]
        if p["units"] <= 2000:
            cover = {}
            for u in range(p["units"]):
                bt, i, j, kb, ke = g.gemm355_unit(a, u)
                cover.setdefault((bt, i, j), []).append((kb, ke))
            assert len(cover) == p["G"], (M, N, K, batch, name, knobs)
            for ranges in cover.values():
                ranges.sort()
                assert ranges[0][0] == 0 and ranges[-1][1] == p["nK"]
                assert all(e0 == b1 for (_, e0), (b1, _) in zip(ranges, ranges[1:]))


def test_plan_reports_efficiency_levers(g):
    """The named ragged and split-K shapes are planned with a persistent tail
    split or a K-split that fills the device."""
    for (M, N, K) in [(4097, 4095, 4104), (256, 256, 65536), (128, 512, 131072), (64, 64, 262144)]:
        a = g.make_args(M, N, K, A=0x10000, B=0x1000000000, C=0x200000000000, cus=256)
        p = g.gemm355_plan(a)
        assert p["split"] > 1 or p["tail_tiles"] > 0
        assert Fraction(p["eta_sched_num"], p["eta_sched_den"]) >= Fraction(95, 100)
    a = g.make_args(4096, 4096, 4096, A=0x10000, B=0x1000000000, C=0x200000000000,
                    dtype=g.BF16_BF16, cus=256)
    p = g.gemm355_plan(a)
    assert (p["T_M"], p["T_N"], p["G"], p["eta_wave_num"], p["eta_wave_den"]) == (256, 256, 256, 1, 1)
    # the large named shapes fill the device to eta_sched >= 0.95 (the tail
    # and long-K shapes through the levers above)
    shapes = [(4000, 4000, 4000, 1, g.BF16_F32), (8192, 8192, 8192, 1, g.E4M3_F32),
              (512, 1024, 4096, 64, g.E4M3_F32)]
    for (M, N, K, batch, dt) in shapes:
        a = g.make_args(M, N, K, A=0x10000, B=0x1000000000, C=0x200000000000, dtype=dt, batch=batch,
                        stride_a=M * K, stride_b=N * K, stride_c=M * N, cus=256)
        p = g.gemm355_plan(a)
        assert Fraction(p["eta_sched_num"], p["eta_sched_den"]) >= Fraction(95, 100), (M, N, K)
    # 1000 x 3000 x 777: 192 tiles of 128 x 128 in one round (eta_sched 3/4)
    # model faster than 752 of 64 x 64 (47/48) by more than the tie band
    p = g.gemm355_plan(g.make_args(1000, 3000, 777, A=0x10000, B=0x1000000000, C=0x200000000000, cus=256))
    assert (p["T_M"], p["T_N"], p["G"]) == (128, 128, 192)
    assert (p["eta_sched_num"], p["eta_sched_den"]) == (3, 4)


def test_plan_fits_short_k_and_narrow_shapes(g):
    """The time model charges a pipeline fill and epilogue per unit a slot
    runs in turn, so the shortest-K product with narrow N goes to 64x64
    tiles with several resident workgroups per compute unit, a narrow
    product with longer K to 256x128 tiles with producer wavefronts (the
    calibration sweep timed that plan at 59.2 us, the best 128x128 one at
    63.6 us), while the square product keeps its 256x256 tile."""
    base = dict(A=0x10000, B=0x1000000000, C=0x200000000000, cus=256)
    p = g.gemm355_plan(g.make_args(100352, 64, 256, dtype=g.BF16_BF16, **base))
    assert (p["T_M"], p["T_N"]) == (64, 64) and p["b"] >= 2
    p = g.gemm355_plan(g.make_args(100352, 128, 1152, dtype=g.BF16_BF16, **base))
    assert (p["T_M"], p["T_N"]) == (256, 128) and g.gemm355_tile_info(p["tile"])["schedule"] == 3
    p = g.gemm355_plan(g.make_args(4096, 4096, 4096, dtype=g.BF16_BF16, **base))
    assert (p["T_M"], p["T_N"], p["grid"], p["split"]) == (256, 256, 256, 1)
    # a 1x1 convolution with 64 output channels: 64x64 tiles, several per CU
    a = g.make_conv_args(32, 56, 56, 256, 64, 1, 1, x=0x10000, w=0x1000000000, y=0x200000000000,
                         dtype=g.BF16_BF16)
    p = g.gemm355_conv2d_plan(a)
    assert (p["T_M"], p["T_N"]) == (64, 64) and p["b"] >= 2


def test_repack_decisions(g):
    """K-contiguous bf16 / 8-bit rows are read in place (K ending inside a
    16-byte chunk plans only tiles that clear the chunk's bytes past K),
    except rows that are not 16-byte aligned in products whose dense-MFMA
    time at peak reaches 10 us; the transposed layouts are repacked, and so
    are block-scaled rows that are not 16-byte aligned, and in-place rows
    with a K tail under a forced tile without the clearing."""
    base = dict(A=0x10000, B=0x1000000000, C=0x200000000000, cus=256)
    p = g.gemm355_plan(g.make_args(1000, 3000, 777, **base))       # rows 2-byte aligned, K tail
    assert p["repack"] == 0 and g.gemm355_tile_info(p["tile"])["stages"] >= 2
    assert g.gemm355_plan(g.make_args(1000, 3000, 776, **base))["repack"] == 0
    # misaligned rows around the threshold: 2 M N K / 2516.6 TFLOP/s = 10 us at M N K = 12.58e9
    assert g.gemm355_plan(g.make_args(2000, 2000, 2001, **base))["repack"] == 0      # 8.0e9
    assert g.gemm355_plan(g.make_args(2500, 2500, 2501, **base))["repack"] == 3      # 15.6e9
    assert g.gemm355_plan(g.make_args(2500, 2500, 2504, **base))["repack"] == 0      # rows 16-byte aligned
    assert g.gemm355_plan(g.make_args(2500, 2500, 2504, lda=2505, **base))["repack"] == 1
    assert g.gemm355_plan(g.make_args(2500, 2500, 2501, dtype=g.E4M3_F32, **base))["repack"] == 0  # fp8 peak twice
    assert g.gemm355_plan(g.make_args(3200, 3200, 3201, dtype=g.E4M3_F32, **base))["repack"] == 3
    # on 64 compute units the same product takes four times as long at peak
    assert g.gemm355_plan(g.make_args(2000, 2000, 2001, **dict(base, cus=64)))["repack"] == 3
    assert g.gemm355_plan(g.make_args(64, 64, 64, layout=g.A_COL_B_COL, **base))["repack"] == 1
    assert g.gemm355_plan(g.make_args(64, 64, 64, layout=g.A_ROW_B_ROW, **base))["repack"] == 2
    b2 = dict(base, A=0x10002)
    assert g.gemm355_plan(g.make_args(64, 64, 64, **b2))["repack"] == 0
    assert g.gemm355_plan(g.make_args(64, 64, 128, dtype=g.E4M3_F32, **base))["repack"] == 0
    assert g.gemm355_plan(g.make_args(64, 64, 120, dtype=g.E4M3_F32, **base))["repack"] == 0
    # a forced tile whose copy schedule does not clear a K tail: repacked
    spread1 = [t for t in range(g.gemm355_num_tiles()) if g.gemm355_tile_info(t)["dtype_class"] == 0
               and g.gemm355_tile_info(t)["op"] == 0 and g.gemm355_tile_info(t)["schedule"] == 1]
    assert g.gemm355_plan(g.make_args(1000, 3000, 777, tile=spread1[0], **base))["repack"] == 3
    assert g.gemm355_plan(g.make_args(1000, 3000, 776, tile=spread1[0], **base))["repack"] == 0
    # block-scaled rows that are not 16-byte aligned are repacked
    mx = dict(base, block_scale_a=0x4000, block_scale_b=0x8000)
    assert g.gemm355_plan(g.make_args(64, 64, 128, dtype=g.MXE4M3_F32, lda=136, **mx))["repack"] == 1


def test_argument_errors(g):
    P = dict(A=0x10000, B=0x1000000000, C=0x200000000000)

    def status(**kw):
        args = dict(P)
        args.update(kw)
        M, N, K = args.pop("M", 64), args.pop("N", 64), args.pop("K", 64)
        try:
            g.gemm355_gemm_ex(g.make_args(M, N, K, **args), stream=0)
            return g.OK
        except g.Gemm355Error as e:
            return e.status

    assert status(M=-1) == g.EINVAL
    assert status(K=-5) == g.EINVAL
    assert status(lda=10) == g.EINVAL
    assert status(ldb=10) == g.EINVAL
    assert status(ldc=10) == g.EINVAL
    assert status(A=None) == g.EINVAL
    assert status(C=None) == g.EINVAL
    assert status(A=0x10001) == g.EALIGN
    assert status(unit_stamps=0x300000000004) == g.EALIGN  # stamps need 8-byte alignment
    assert status(C=0x200000000002) == g.EALIGN            # fp32 C
    assert status(scale_a=0x3001) == g.EALIGN
    assert status(dtype=20) == g.EINVAL
    # MX FP6: native layout, leading dimensions multiples of 64, K a multiple of 128
    FP6 = dict(dtype=g.MXFP6_E2M3_F32, block_scale_a=0x300000000000, block_scale_b=0x380000000000)
    g.gemm355_plan(g.make_args(64, 64, 128, **P, **FP6))      # valid
    assert status(K=64, **FP6) == g.EUNSUPPORTED
    assert status(K=128, lda=160, **FP6) == g.EUNSUPPORTED
    assert status(K=128, layout=g.A_ROW_B_ROW, ldb=64, **FP6) == g.EUNSUPPORTED
    # MX FP4: native layout, even leading dimensions, K a multiple of 256
    FP4 = dict(dtype=g.MXFP4_F32, block_scale_a=0x300000000000, block_scale_b=0x380000000000)
    g.gemm355_plan(g.make_args(64, 64, 256, **P, **FP4))      # valid
    assert status(K=128, **FP4) == g.EUNSUPPORTED
    assert status(K=256, lda=258 + 1, **FP4) == g.EUNSUPPORTED
    assert status(K=256, lda=264, **FP4) == g.EUNSUPPORTED     # 132-byte rows: not 16-byte aligned
    assert status(K=256, layout=g.A_COL_B_COL, lda=64, **FP4) == g.EUNSUPPORTED
    assert status(K=256, A=0x10008, **FP4) == g.EUNSUPPORTED   # would need a repack
    # block-scaled dtypes: scales required (and only there), K a multiple of 128
    BS = dict(block_scale_a=0x300000000000, block_scale_b=0x380000000000)
    g.gemm355_plan(g.make_args(64, 64, 128, dtype=g.MXE4M3_F32, **P, **BS))   # valid
    assert status(dtype=g.MXE4M3_F32, K=128) == g.EINVAL
    assert status(dtype=g.MXE4M3_F32, K=128, block_scale_a=BS["block_scale_a"]) == g.EINVAL
    assert status(dtype=g.MXE4M3_F32, K=64, **BS) == g.EUNSUPPORTED
    assert status(dtype=g.MXE4M3_F32, K=128, block_scale_a=0x300000000002,
                  block_scale_b=BS["block_scale_b"]) == g.EALIGN
    assert status(dtype=g.MXE4M3_F32, K=128, block_scale_a=0x200000000000 + 256,
                  block_scale_b=BS["block_scale_b"]) == g.EINVAL   # scales overlap C
    g.gemm355_plan(g.make_args(64, 64, 0, dtype=g.MXE5M2_BF16, **P))  # K = 0: C = 0, no scales read
    assert status(dtype=g.E4M3_F32, **BS) == g.EINVAL        # block scales for a per-tensor dtype
    assert status(dtype=g.MXE4M3_F32, K=128, tile=3, **BS) == g.EINVAL   # tile of another class
    assert status(layout=9) == g.EINVAL
    assert status(tile=99) == g.EINVAL
    assert status(tile=3) == g.EINVAL                      # E4M3 tile for bf16 inputs
    assert status(persistent=2) == g.EINVAL
    assert status(split_k=-1) == g.EINVAL
    assert status(batch=0) == g.EINVAL
    assert status(cus=-3) == g.EINVAL
    assert status(C=0x10000 + 64) == g.EINVAL              # C overlaps A
    assert status(lda=(1 << 24)) == g.EUNSUPPORTED         # 32-bit tile offsets
    # split-K needs scratch: a caller workspace that is too small
    assert status(K=65536, split_k=8, workspace=0x300000000000, workspace_bytes=16) == g.ENOMEM
    assert status(K=65536, split_k=8, workspace=0x300000000010, workspace_bytes=1 << 30) == g.EALIGN
    # nothing to do: M or N zero is accepted without touching the device
    assert status(M=0) == g.OK
    assert status(N=0, C=None) == g.OK
    assert g.gemm355_status_string(g.ENOMEM).startswith("workspace")


def test_scratch_limit_roundtrip(g):
    """The library-scratch cap is a process-wide value: each set returns the
    previous one, the default is no cap."""
    prev = g.gemm355_set_scratch_limit(12345)
    try:
        assert prev == g.SCRATCH_UNLIMITED
        assert g.gemm355_set_scratch_limit(0) == 12345
    finally:
        assert g.gemm355_set_scratch_limit(prev) == 0


def test_quantize_argument_errors(g):
    """Argument checks of the quantiser run before anything touches a device."""
    X, Q, S = 0x10000, 0x1000000000, 0x200000000000

    def status(**kw):
        a = dict(x=X, n=1024, batch=1, src=g.SRC_F32, fmt=g.FP8_E4M3, q=Q, scale=S)
        a.update(kw)
        try:
            g.gemm355_quantize(a["x"], a["n"], a["batch"], a["src"], a["fmt"], a["q"], a["scale"], stream=0)
            return g.OK
        except g.Gemm355Error as e:
            return e.status

    assert status(n=-1) == g.EINVAL
    assert status(batch=0) == g.EINVAL
    assert status(src=2) == g.EINVAL
    assert status(fmt=5) == g.EINVAL
    assert status(scale=None) == g.EINVAL
    assert status(x=None) == g.EINVAL
    assert status(q=None) == g.EINVAL
    assert status(scale=S + 2) == g.EALIGN
    assert status(x=X + 2) == g.EALIGN                       # fp32 input
    assert status(q=X + 100) == g.EINVAL                     # codes overlap the input
    assert status(scale=X + 64) == g.EINVAL                  # scales overlap the input
    assert status(n=1 << 40) == g.EUNSUPPORTED
    assert status(n=1 << 20, batch=1 << 21) == g.EUNSUPPORTED


def test_tile_table(g):
    n = g.gemm355_num_tiles()
    assert n >= 6
    seen = set()
    for t in range(n):
        info = g.gemm355_tile_info(t)
        cls = info["dtype_class"]
        row_bytes = info["T_K"] // 2 if cls == 3 else info["T_K"] * (1 if cls else 2)
        assert row_bytes in (64, 128)
        # block-scaled tiles keep one dword of E8M0 scales (four 32-value
        # blocks) per 128 values, per row and stage
        scale_bytes = {2: 4, 3: 8, 4: 4}.get(cls, 0)
        # copy schedules 5 and 6 keep one more B tile than A tiles
        b_stages = info["stages"] + (1 if info["schedule"] in (5, 6) else 0)
        assert info["lds_bytes"] == (info["stages"] * info["T_M"] + b_stages * info["T_N"]) * (row_bytes + scale_bytes)
        assert info["schedule"] in range(7)
        if info["schedule"] == 6:
            # the ping-pong pairs the two block rows of 2 x 4 wavefronts
            assert info["waves"] == 8 and info["stages"] == 2
        assert info["lds_bytes"] <= 160 * 1024
        seen.add((info["dtype_class"], info["T_M"], info["T_N"]))
    assert (0, 256, 256) in seen and (1, 256, 256) in seen and (2, 256, 256) in seen and (3, 256, 256) in seen
    with pytest.raises(g.Gemm355Error):
        g.gemm355_tile_info(n)


def test_main_loop_uses_mfma(g, tmp_path):
    """The compiler emitted the matrix-core instruction family for every
    main-loop instantiation (bf16 and each 8-bit format pair), not a scalar
    fallback, with the operand-format fields of the pair."""
    from dense_tiled_gemm_fp8_amd import build
    asm = open(build.device_asm("kernels.hip")).read()
    bodies = re.split(r"\n(?=_ZN4g35516gemm_tile_kernel\w+:)", asm)
    kernels = [b for b in bodies if re.match(r"_ZN4g35516gemm_tile_kernel\w+:", b)]
    n8 = sum(g.gemm355_tile_info(t)["dtype_class"] in (1, 2, 4) for t in range(g.gemm355_num_tiles()))
    assert len(kernels) == g.gemm355_num_tiles() + 2 * n8      # three format pairs per 8-bit tile
    for body in kernels:
        name = body.split(":")[0]
        targs = [int(v) for v in re.findall(r"Li(\d+)E", name)]
        el, mi, fmt = targs[2], targs[-2], targs[-1]        # element class, MFMA block edge, format pair
        fp8 = el != 0
        want = {(1, 32): "v_mfma_f32_32x32x64_f8f6f4", (0, 32): "v_mfma_f32_32x32x16_bf16",
                (1, 16): "v_mfma_f32_16x16x128_f8f6f4", (0, 16): "v_mfma_f32_16x16x32_bf16",
                (2, 32): "v_mfma_scale_f32_32x32x64_f8f6f4", (3, 32): "v_mfma_scale_f32_32x32x64_f8f6f4",
                (4, 32): "v_mfma_scale_f32_32x32x64_f8f6f4"}[(el, mi)]
        code = body.split("s_endpgm")[0]
        lines = [l for l in code.splitlines() if want in l]
        assert lines, name
        if el == 3:
            # FP4 (E2M1) is format 4 for both operands
            assert all("cbsz:4" in l and "blgp:4" in l for l in lines), name
        elif el == 4:
            # FP6: E2M3 format 2, E3M2 format 3
            assert all(("cbsz:3" if fmt == 1 else "cbsz:2") in l for l in lines), name
            assert all(("blgp:3" if fmt >= 1 else "blgp:2") in l for l in lines), name
        elif fp8:
            # E4M3 is format 0 (no modifier printed), E5M2 format 1
            assert all(("cbsz:1" in l) == (fmt == 1) for l in lines), name
            assert all(("blgp:1" in l) == (fmt >= 1) for l in lines), name
        else:
            assert fmt == 0
        # no register spills anywhere in the kernel (a spill reloaded in the
        # main loop or prologue costs far more than the instructions it saves)
        m = re.search(r"; ScratchSize: (\d+)", body)
        assert m and int(m.group(1)) == 0, (name, m and m.group(1))


def test_struct_layout_matches_header(g, tmp_path):
    """The binding's ctypes structures have the header's layout: a C
    program built from include/gemm355.h prints sizeof and every field's
    offsetof, which must equal ctypes' view."""
    import ctypes
    import subprocess
    hdr = os.path.join(ROOT, "include")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gemm355.h"', "int main(void) {"]
    for cls, cname in ((g.gemm355_args, "gemm355_args"), (g.gemm355_plan_t, "gemm355_plan_t")):
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (cname, cname))
        for name, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, name, cname, name))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", hdr, str(src), "-o", str(exe)])
    out = dict(l.rsplit(" ", 1) for l in subprocess.check_output([str(exe)]).decode().split("\n") if l)
    for cls, cname in ((g.gemm355_args, "gemm355_args"), (g.gemm355_plan_t, "gemm355_plan_t")):
        assert int(out[cname]) == ctypes.sizeof(cls), cname
        for name, _ in cls._fields_:
            assert int(out["%s.%s" % (cname, name)]) == getattr(cls, name).offset, (cname, name)


def test_conv_plan_and_argument_errors(g):
    """The convolution's implicit product: M = N P Q, N = K, K = R S C with
    the library's output size; argument checks before any device work."""
    X, W, Y = 0x10000, 0x1000000000, 0x200000000000

    def args(**kw):
        a = dict(N=4, H=30, W=30, C=64, K=96, R=3, S=3, x=X, w=W, y=Y, pad_h=1, pad_w=1, cus=256)
        a.update(kw)
        return g.make_conv_args(**a)

    p = g.gemm355_conv2d_plan(args())
    assert (p["T_M"], p["T_N"], p["T_K"]) != (0, 0, 0)
    P, Q = g.gemm355_conv2d_out_size(args())
    assert (P, Q) == (30, 30) == oc.out_size(30, 30, 3, 3, 1, 1, 1, 1, 1, 1)
    assert p["G"] == bk.tile_grid(4 * P * Q, 96, p["T_M"], p["T_N"])
    assert p["nK"] == bk.ceil_div(9 * 64, p["T_K"])
    assert g.gemm355_tile_info(p["tile"])["op"] == 1
    p2 = g.gemm355_conv2d_plan(args(stride_h=2, stride_w=3, dil_h=2, pad_h=0, pad_w=0))
    P2, Q2 = g.gemm355_conv2d_out_size(args(stride_h=2, stride_w=3, dil_h=2, pad_h=0, pad_w=0))
    assert (P2, Q2) == oc.out_size(30, 30, 3, 3, 0, 0, 2, 3, 2, 1)
    assert p2["G"] == bk.tile_grid(4 * P2 * Q2, 96, p2["T_M"], p2["T_N"])

    def status(**kw):
        try:
            g.gemm355_conv2d(args(**kw), stream=0)
            return g.OK
        except g.Gemm355Error as e:
            return e.status

    assert status(C=3) == g.EUNSUPPORTED                    # 64-channel K-tiles
    assert status(H=2, pad_h=0) == g.EINVAL                 # P < 1
    assert status(stride_h=0) == g.EINVAL
    assert status(dil_w=0) == g.EINVAL
    assert status(pad_w=-1) == g.EINVAL
    assert status(N=0) == g.EINVAL
    assert status(dtype=g.E4M3_F32) == g.EUNSUPPORTED
    assert status(dtype=99) == g.EINVAL
    assert status(x=None) == g.EINVAL
    assert status(y=X + 64) == g.EINVAL                     # output overlaps the images
    assert status(x=X + 8) == g.EUNSUPPORTED                 # pixels not 16-byte aligned
    assert status(tile=0) == g.EINVAL                       # a matrix-product tile
    assert status(N=1 << 12, H=1 << 10, W=1 << 10) == g.EUNSUPPORTED   # images beyond 2 GiB
    with pytest.raises(g.Gemm355Error):
        g.gemm355_conv2d_plan(None)
