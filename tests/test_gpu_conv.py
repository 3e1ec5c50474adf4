"""GPU parity for the implicit-GEMM convolution (gemm355_conv2d) against
oracle/conv.py: bf16 NHWC images and KRSC filters, fp32 accumulate, fp32 or
bf16 output NPQK, within |y_gpu - y_ref| <= 1e-3 W + 1e-6 (W = sum |x w|);
bit-exact on small integers; padding, stride, dilation, ragged output
pixels and channels, every convolution tile, split-K and the persistent
grid."""
import numpy as np
import pytest
import torch

from dense_tiled_gemm_fp8_amd import gemm355 as g
from dense_tiled_gemm_fp8_amd import inputs
from oracle import conv as oc
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

CONV_TILES = [t for t in range(g.gemm355_num_tiles()) if g.gemm355_tile_info(t)["op"] == 1]


def run_conv(x, w, ph=0, pw=0, sh=1, sw=1, dh=1, dw=1, out="f32", **knobs):
    N, Hh, W, C = x.shape
    K, R, S, _ = w.shape
    xd, wd = H.dev(x), H.dev(w)
    a = g.make_conv_args(N, Hh, W, C, K, R, S, x=xd, w=wd, pad_h=ph, pad_w=pw, stride_h=sh,
                         stride_w=sw, dil_h=dh, dil_w=dw, dtype=g.BF16_BF16 if out == "bf16" else g.BF16_F32,
                         **knobs)
    P, Q = g.gemm355_conv2d_out_size(a)
    y = torch.full((N, P, Q, K), float("nan"), dtype=torch.bfloat16 if out == "bf16" else torch.float32,
                   device="cuda")
    a.y = y.data_ptr()
    g.gemm355_conv2d(a)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


CASES = [
    # N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw
    (2, 9, 11, 64, 70, 3, 3, 1, 1, 1, 1, 1, 1),
    (1, 17, 13, 128, 64, 3, 3, 1, 1, 2, 2, 1, 1),
    (3, 10, 10, 64, 33, 3, 2, 2, 0, 1, 2, 2, 1),
    (1, 7, 30, 192, 130, 1, 5, 0, 2, 1, 1, 1, 3),
    (4, 6, 6, 64, 257, 1, 1, 0, 0, 1, 1, 1, 1),
    (1, 20, 20, 64, 64, 7, 7, 3, 3, 2, 2, 1, 1),
]


@pytest.mark.parametrize("case", CASES)
def test_conv_full(case):
    N, Hh, W, C, K, R, S, ph, pw, sh, sw, dh, dw = case
    x, w = inputs.conv_operands(N, Hh, W, C, K, R, S, "uniform", 900 + sum(case), 901 + N)
    y_ref, mag = oc.conv2d(x, w, ph, pw, sh, sw, dh, dw)
    for tile in [-1] + CONV_TILES:
        for out in ("f32", "bf16"):
            H.say("conv", case, "tile", tile, out)
            y = run_conv(x, w, ph, pw, sh, sw, dh, dw, out=out, tile=tile)
            if out == "f32":
                H.check(y, y_ref, mag, "bf16", "conv %s tile %d" % (case, tile))
            else:
                ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y_ref), 2.0 ** -126))) - 7)
                assert np.all(np.abs(y - y_ref) <= 1e-3 * mag + 1e-6 + ulp / 2), (case, tile)


def test_conv_exact_integers_split_and_persistent():
    N, Hh, W, C, K, R, S = 2, 12, 9, 128, 96, 3, 3
    gen = inputs.rng(77)
    x = inputs.small_int_codes(gen, (N, Hh, W, C), "bf16")
    w = inputs.small_int_codes(gen, (K, R, S, C), "bf16")
    y_ref, _ = oc.conv2d(x, w, 1, 2, 1, 2, 1, 1)
    for tile in CONV_TILES:
        for knobs in (dict(split_k=1, persistent=0), dict(split_k=3), dict(persistent=1)):
            H.say("conv ints tile", tile, knobs)
            y = run_conv(x, w, 1, 2, 1, 2, out="f32", tile=tile, **knobs)
            assert np.array_equal(y, y_ref), (tile, knobs)


def test_conv_resnet_layer_sampled():
    """A 3x3 layer of 56 x 56 x 128 images, batch 16 (M = 50176 output
    pixels, K = 1152): sampled outputs, corners and edges included."""
    N, Hh, W, C, K, R, S = 16, 56, 56, 128, 128, 3, 3
    x, w = inputs.conv_operands(N, Hh, W, C, K, R, S, "normal", 950, 951)
    H.say("conv resnet layer")
    y = run_conv(x, w, 1, 1)
    gen = inputs.rng(12)
    idx = np.stack([gen.integers(0, N, 2000), gen.integers(0, 56, 2000), gen.integers(0, 56, 2000),
                    gen.integers(0, K, 2000)], axis=1)
    edges = np.array([[0, 0, 0, 0], [N - 1, 55, 55, K - 1], [3, 0, 55, 7], [9, 55, 0, 100]])
    idx = np.concatenate([idx, edges])
    ref, mag = oc.conv2d_entries(x, w, idx, 1, 1)
    H.check(y[tuple(idx.T)], ref, mag, "bf16", "conv resnet sampled")
