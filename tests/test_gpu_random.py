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


@pytest.mark.parametrize("block", range(8))
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


LAYOUTS = [g.A_ROW_B_COL, g.A_ROW_B_ROW, g.A_COL_B_COL, g.A_COL_B_ROW]


def _stored(codes_rows_by_k, k_contig, ld, off, fill):
    """A logical rows x K operand (codes) laid out K-contiguous (rows of ld
    elements) or transposed (K rows of ld elements), starting `off` elements
    into a buffer whose every other element is a NaN code."""
    rows, K = codes_rows_by_k.shape
    st = codes_rows_by_k if k_contig else np.ascontiguousarray(codes_rows_by_k.T)
    n_rows, n_cols = st.shape
    buf = np.full(off + n_rows * ld + 64, fill, dtype=st.dtype)
    buf[off:off + n_rows * ld].reshape(n_rows, ld)[:, :n_cols] = st
    return H.dev(buf)[off:]


@pytest.mark.parametrize("block", range(5))
def test_random_layouts_exact(block):
    """Random storage layout (the three non-native ones are repacked on the
    device), leading dimensions padded past the matrix with NaN codes,
    operands starting off 16-byte boundaries, fp32 or bf16 C (bf16 against
    the exact result rounded to nearest even), forced tiles and knobs:
    exact integers, bit for bit."""
    import torch
    rnd = random.Random(2000 + block)
    for case in range(30):
        fmt = rnd.choice(["bf16", "e4m3", "e5m2", "e4m3e5m2"])
        M, N, K = rnd.randint(1, 400), rnd.randint(1, 400), rnd.randint(1, 700)
        layout = rnd.choice(LAYOUTS)
        a_row = layout in (g.A_ROW_B_COL, g.A_ROW_B_ROW)
        b_col = layout in (g.A_ROW_B_COL, g.A_COL_B_COL)
        pad_a, pad_b = rnd.choice([0, 0, 1, 3, 8, 17]), rnd.choice([0, 0, 1, 3, 8, 17])
        off_a, off_b = rnd.choice([0, 0, 1, 5]), rnd.choice([0, 0, 1, 5])
        out = rnd.choice(["f32", "bf16"])
        tile = rnd.choice(TILES[CLASS[fmt]] + [-1, -1])
        knobs = rnd.choice(KNOBS)
        ops = H.exact_ops(M, N, K, fmt, 60000 + 100 * block + case)
        fa, fb = H.elem_formats(fmt)
        nan = {"bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F), "e5m2": np.uint8(0x7F)}
        lda = (K if a_row else M) + pad_a
        ldb = (K if b_col else N) + pad_b
        A_dev = _stored(ops.A, a_row, lda, off_a, nan[fa])
        B_dev = _stored(ops.B, b_col, ldb, off_b, nan[fb])
        what = "layout case %d.%d: %s M=%d N=%d K=%d layout=%d lda=%d ldb=%d off=%d,%d out=%s tile=%d %s" % (
            block, case, fmt, M, N, K, layout, lda, ldb, off_a, off_b, out, tile, knobs)
        H.say(what)
        C = H.run(ops, out=out, layout=layout, A_dev=A_dev, B_dev=B_dev, lda=lda, ldb=ldb, tile=tile, **knobs)
        ref, _ = H.oracle_full(ops, 0, alpha=1.0)
        if out == "bf16":
            ref = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
        assert np.array_equal(C, ref), what


@pytest.mark.parametrize("block", range(4))
def test_random_convolutions_exact(block):
    """Random implicit-GEMM convolutions: image count and size, channels (64
    to 256), filter count and size, padding, stride and dilation, every
    convolution tile or the planner's, split and persistence knobs, fp32 or
    bf16 output, small integer images and filters: bit for bit against the
    oracle's convolution (bf16 output: the exact result rounded to nearest
    even)."""
    import torch
    from dense_tiled_gemm_fp8_amd import inputs
    from oracle import conv as oc
    conv_tiles = [t for t in range(g.gemm355_num_tiles()) if g.gemm355_tile_info(t)["op"] == 1]
    rnd = random.Random(3000 + block)
    done = 0
    while done < 20:
        N, Hh, W = rnd.randint(1, 4), rnd.randint(1, 24), rnd.randint(1, 24)
        C, K = rnd.choice([64, 128, 192, 256]), rnd.randint(1, 300)
        R, S = rnd.randint(1, 5), rnd.randint(1, 5)
        ph, pw = rnd.randint(0, 3), rnd.randint(0, 3)
        sh, sw, dh, dw = rnd.choice([1, 1, 2, 3]), rnd.choice([1, 1, 2, 3]), rnd.choice([1, 1, 2]), rnd.choice([1, 1, 2])
        P, Q = oc.out_size(Hh, W, R, S, ph, pw, sh, sw, dh, dw)
        if P < 1 or Q < 1:
            continue
        tile = rnd.choice(conv_tiles + [-1, -1])
        knobs = rnd.choice(KNOBS)
        out = rnd.choice(["f32", "bf16"])
        gen = inputs.rng(70000 + 100 * block + done)
        x = inputs.small_int_codes(gen, (N, Hh, W, C), "bf16")
        w = inputs.small_int_codes(gen, (K, R, S, C), "bf16")
        what = "conv case %d.%d: N=%d %dx%dx%d K=%d %dx%d pad %d,%d stride %d,%d dil %d,%d out=%s tile=%d %s" % (
            block, done, N, Hh, W, C, K, R, S, ph, pw, sh, sw, dh, dw, out, tile, knobs)
        H.say(what)
        # the device copies stay referenced until the call has run (make_conv_args keeps raw pointers)
        xd, wd = H.dev(x), H.dev(w)
        a = g.make_conv_args(N, Hh, W, C, K, R, S, x=xd, w=wd, pad_h=ph, pad_w=pw, stride_h=sh,
                             stride_w=sw, dil_h=dh, dil_w=dw, dtype=g.BF16_BF16 if out == "bf16" else g.BF16_F32,
                             tile=tile, **knobs)
        y = torch.full((N, P, Q, K), float("nan"), dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                       device="cuda")
        a.y = y.data_ptr()
        g.gemm355_conv2d(a)
        torch.cuda.synchronize()
        got = y.float().cpu().numpy().astype(np.float64)
        del xd, wd
        ref, _ = oc.conv2d(x, w, ph, pw, sh, sw, dh, dw)
        if out == "bf16":
            ref = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
        assert np.array_equal(got, ref), what
        done += 1
