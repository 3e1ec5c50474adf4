"""GPU parity for the FP8 pair of the Hopper row of the input/accumulate
table (page "The Tensor Core"): E5M2 operands and mixed E4M3 x E5M2 operands
through the MFMA main loop, and the on-device per-tensor quantiser whose
overhead page "10. Tensor Cores, shapes, and tile alignment" (section
"Practical shape sweep") asks to include.

* products: element by element against the binary64 oracle within
  2e-2 * W, and bit-exact on small integers through every 8-bit tile;
* quantiser: codes and scales bit-identical to oracle/quant.py (an integer
  decision taken in binary32 on both sides) for fp32 and bf16 sources,
  both formats, aligned and misaligned buffers, empty tensors, batches;
* end to end: quantise A and B on the device, multiply with the device
  scales, compare with the oracle's product of the oracle's codes.
"""
import numpy as np
import pytest
import torch

from dense_tiled_gemm_fp8_amd import gemm355 as g
from dense_tiled_gemm_fp8_amd import inputs
from oracle import quant as oq
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

_TILES = [(t, g.gemm355_tile_info(t)["dtype_class"]) for t in range(g.gemm355_num_tiles())
          if g.gemm355_tile_info(t)["op"] == 0]
F8_TILES = [t for t, c in _TILES if c == 1]
FMT_OF = {"e4m3": g.FP8_E4M3, "e5m2": g.FP8_E5M2}


def int_ops(M, N, K, fmt, seed, batch=0):
    ga, gb = inputs.rng(seed), inputs.rng(seed + 1)
    fa = "e5m2" if fmt == "e5m2" else "e4m3"
    fb = "e4m3" if fmt == "e4m3" else "e5m2"
    nb = max(batch, 1)
    A = np.stack([inputs.small_int_codes(ga, (M, K), fa) for _ in range(nb)])
    B = np.stack([inputs.small_int_codes(gb, (N, K), fb) for _ in range(nb)])
    if not batch:
        A, B = A[0], B[0]
    return inputs.Operands(M, N, K, fmt, A, B, [1.0] * nb, [1.0] * nb, (seed, seed + 1))


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3e5m2"])
@pytest.mark.parametrize("shape", [(300, 520, 256), (257, 129, 144), (70, 90, 77), (1, 1, 16)])
def test_fp8_formats_ragged_full(fmt, shape):
    M, N, K = shape
    ops = inputs.make_operands(M, N, K, fmt, "normal", 500 + M + K, 501 + N)
    C_ref, W = H.oracle_full(ops)
    for tile in (-1, 3, 4, 5, 12, 17, 22):
        for out in ("f32", "bf16"):
            H.say(fmt, "tile", tile, shape, out)
            C = H.run(ops, out=out, tile=tile)
            if out == "f32":
                H.check(C, C_ref, W, fmt, "%s tile %d %s" % (fmt, tile, shape))
            else:
                # bf16 output: add half an ulp of bf16 at |C_ref| to the bound
                ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(C_ref), 2.0 ** -126))) - 7)
                assert np.all(np.abs(C - C_ref) <= 2e-2 * W + ulp / 2), (fmt, tile, shape)


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3e5m2"])
def test_fp8_formats_exact_integers_every_tile(fmt):
    M, N, K, batch = 200, 170, 384, 2
    ops = int_ops(M, N, K, fmt, 61, batch=batch)
    refs = [H.oracle_full(ops, bi, alpha=1.0)[0] for bi in range(batch)]
    for tile in F8_TILES:
        for knobs in (dict(split_k=1, persistent=0), dict(split_k=3), dict(persistent=1)):
            H.say(fmt, "ints tile", tile, knobs)
            C = H.run(ops, out="f32", tile=tile, **knobs)
            for bi in range(batch):
                assert np.array_equal(C[bi], refs[bi]), (fmt, tile, knobs, bi)


def _quantize_dev(x_np, src, fmt, n, batch, x_off=0, q_off=0):
    """Run the device quantiser on x (fp32 numpy, converted to `src`), with
    the input and output starting x_off / q_off elements into their buffers.
    Returns (codes, scales, the binary32 values actually quantised)."""
    if src == "bf16":
        xt = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).to(torch.bfloat16)
        x_used = xt.float().numpy()
        buf = torch.zeros(x_off + n * batch + 8, dtype=torch.bfloat16)
    else:
        xt = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32))
        x_used = xt.numpy()
        buf = torch.zeros(x_off + n * batch + 8, dtype=torch.float32)
    buf[x_off:x_off + n * batch] = xt.reshape(-1)
    xd = buf.cuda()
    qd = torch.full((q_off + n * batch + 8,), 0xA5, dtype=torch.uint8, device="cuda")
    sd = torch.full((batch,), -1.0, dtype=torch.float32, device="cuda")
    g.gemm355_quantize(xd.data_ptr() + x_off * xd.element_size(), n, batch,
                       g.SRC_BF16 if src == "bf16" else g.SRC_F32, FMT_OF[fmt],
                       qd.data_ptr() + q_off, sd)
    torch.cuda.synchronize()
    q = qd.cpu().numpy()
    assert np.all(q[:q_off] == 0xA5) and np.all(q[q_off + n * batch:] == 0xA5)
    return q[q_off:q_off + n * batch], sd.cpu().numpy(), x_used.reshape(-1)


def _special_values(fmt, g_):
    F = oq.FMAX[fmt]
    vals, _ = oq._table(fmt)
    mids = ((vals[:-1] + vals[1:]) / 2)
    x = np.concatenate([g_.standard_normal(3000) * 5, [0.0, -0.0, 1e-30, -1e-30],
                        mids[:40] * 3.0, -mids[-10:] * 0.01, [F / 2, -F / 3]])
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_bit_exact(fmt, src):
    g_ = np.random.default_rng(7)
    cases = [(1, 1, 0, 0), (7, 1, 0, 0), (8, 1, 0, 0), (1000, 3, 0, 0), (4099, 2, 1, 3),
             (8192 * 3 + 8, 1, 0, 0), (1 << 20, 2, 0, 0), (0, 2, 0, 0)]
    for n, batch, xo, qo in cases:
        if n == 0:
            x = np.zeros(0, np.float32)
        elif n < 10000:
            x = np.resize(_special_values(fmt, g_), n * batch) * g_.uniform(0.1, 10)
        else:
            x = g_.standard_normal(n * batch).astype(np.float32) * 3
        H.say("quantize", fmt, src, "n", n, "batch", batch, "offsets", xo, qo)
        q, s, xu = _quantize_dev(x, src, fmt, n, batch, xo, qo)
        qref, sref = oq.quantize_batch(xu, n, batch, fmt) if n else (np.zeros(0, np.uint8), np.ones(batch, np.float32))
        assert np.array_equal(s, sref), (s, sref)
        bad = np.flatnonzero(q != qref)
        assert bad.size == 0, "%d codes differ; first at %d: x %r gpu %#x oracle %#x" % (
            bad.size, bad[0], float(xu[bad[0]]), int(q[bad[0]]), int(qref[bad[0]]))
    # exact ties: with amax == F the scale is exactly 1 and every midpoint
    # between neighbouring codes reaches the encoder unchanged
    vals, _ = oq._table(fmt)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    if src == "bf16":
        mids = mids[torch.from_numpy(mids).to(torch.bfloat16).float().numpy() == mids]
    x = np.concatenate([[oq.FMAX[fmt]], mids, -mids]).astype(np.float32)
    H.say("quantize ties", fmt, src, "n", x.size)
    q, s, xu = _quantize_dev(x, src, fmt, x.size, 1)
    qref, sref = oq.quantize(xu, fmt)
    assert s[0] == 1.0 and sref == 1.0
    assert np.array_equal(q, qref)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_then_gemm_end_to_end(fmt):
    """bf16 operands quantised on the device, multiplied with the device
    scales: the codes and scales equal the oracle's, and the product
    matches the oracle's product of them."""
    M, N, K = 640, 384, 1024
    g_ = np.random.default_rng(71)
    xa = g_.standard_normal((M, K)).astype(np.float32)
    xb = g_.standard_normal((N, K)).astype(np.float32) * 0.01
    qa, sa, ua = _quantize_dev(xa, "bf16", fmt, M * K, 1)
    qb, sb, ub = _quantize_dev(xb, "bf16", fmt, N * K, 1)
    ra, rsa = oq.quantize(ua, fmt)
    rb, rsb = oq.quantize(ub, fmt)
    assert np.array_equal(qa, ra) and np.array_equal(qb, rb)
    assert sa[0] == rsa and sb[0] == rsb
    ops = inputs.Operands(M, N, K, fmt, qa.reshape(M, K), qb.reshape(N, K), [float(rsa)], [float(rsb)])
    C_ref, W = H.oracle_full(ops)
    # the device path: codes and scales stay on the device
    Ad = torch.from_numpy(qa).cuda()
    Bd = torch.from_numpy(qb).cuda()
    sad = torch.tensor([sa[0]], dtype=torch.float32, device="cuda")
    sbd = torch.tensor([sb[0]], dtype=torch.float32, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    dt = g.E4M3_F32 if fmt == "e4m3" else g.E5M2_F32
    g.gemm355_gemm_ex(g.make_args(M, N, K, A=Ad, B=Bd, C=C, dtype=dt, scale_a=sad, scale_b=sbd))
    torch.cuda.synchronize()
    H.check(C.cpu().numpy().astype(np.float64), C_ref, W, fmt, "quantise + gemm %s" % fmt)
    # and the product approximates the unquantised one
    exact = (ua.reshape(M, K).astype(np.float64) @ ub.reshape(N, K).astype(np.float64).T)
    rel = np.linalg.norm(C.cpu().numpy() - exact) / np.linalg.norm(exact)
    H.say(fmt, "relative error of the quantised product", rel)
    assert rel < (0.05 if fmt == "e4m3" else 0.15)
