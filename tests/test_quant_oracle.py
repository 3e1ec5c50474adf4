"""Pins for the quantisation oracle (oracle/quant.py), against what the
formats' definitions and an independent library fix:

* the nearest-code encoder against torch's CPU casts to float8_e4m3fn and
  float8_e5m2 (round to nearest, ties to even) on random values and on every
  exact midpoint between neighbouring codes (library special case);
* round trip: every finite code decodes to a value that encodes back to it;
* monotonicity of the encoder, and the error bound |t - dec(q)| <= half the
  gap between the neighbouring codes around t;
* the scale: s == binary32(amax / F), the element of largest magnitude maps
  to the largest finite code, an all-zero tensor gives s = 1 and zero codes;
* a mutation check: an encoder with ties away from zero, or one that
  multiplies by F instead of dividing by it, fails these pins.

The formats (the FP8 pair of the Hopper row of the input/accumulate table on
page "The Tensor Core"): E4M3FN with bias 7 and largest finite 448; E5M2 with
bias 15 and largest finite 57344.
"""
import numpy as np
import pytest
import torch

from oracle import quant, reference

TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FMTS = ("e4m3", "e5m2")


def torch_encode(t, fmt):
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(TORCH[fmt]).view(torch.uint8).numpy()


def decode(codes, fmt):
    return reference.decode_e4m3(codes) if fmt == "e4m3" else reference.decode_e5m2(codes)


def test_e5m2_decode_exhaustive():
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ours = reference.decode_e5m2(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 6                                  # S.11111.{01,10,11}
    hand = {0x7B: 57344.0, 0xFB: -57344.0, 0x3C: 1.0, 0x04: 2.0 ** -14, 0x01: 2.0 ** -16,
            0x03: 3 * 2.0 ** -16, 0x7C: np.inf, 0xFC: -np.inf, 0x40: 2.0, 0x80: -0.0}
    for c, v in hand.items():
        assert reference.decode_e5m2(np.array([c], dtype=np.uint8))[0] == v


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_matches_torch_random(fmt):
    F = quant.FMAX[fmt]
    g = np.random.default_rng(11)
    x = np.concatenate([g.standard_normal(100000) * F / 8, g.uniform(-F, F, 20000),
                        g.standard_normal(20000) * 2.0 ** -12, [0.0, -0.0, F, -F]])
    x = np.clip(x, -F, F).astype(np.float32)
    assert np.array_equal(quant.encode(x, fmt), torch_encode(x, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_ties_to_even(fmt):
    vals, cs = quant._table(fmt)
    mids = (vals[:-1] + vals[1:]) / 2
    m32 = mids.astype(np.float32)
    exact = m32.astype(np.float64) == mids
    assert exact.sum() > 100
    got = quant.encode(m32[exact], fmt)
    assert np.array_equal(got, torch_encode(m32[exact], fmt))
    assert np.all(got % 2 == 0)
    assert np.array_equal(quant.encode(-m32[exact], fmt), got | 0x80)


@pytest.mark.parametrize("fmt", FMTS)
def test_round_trip_and_bounds(fmt):
    vals, cs = quant._table(fmt)
    assert np.array_equal(quant.encode(vals.astype(np.float32), fmt), cs)
    assert np.array_equal(quant.encode(-vals.astype(np.float32), fmt), cs | 0x80)
    g = np.random.default_rng(5)
    t = np.sort(np.clip(g.standard_normal(50000) * quant.FMAX[fmt] / 16, 0, quant.FMAX[fmt])).astype(np.float32)
    q = quant.encode(t, fmt)
    assert np.all(np.diff(q.astype(np.int32)) >= 0)                 # monotone
    d = decode(q, fmt)
    idx = np.clip(np.searchsorted(vals, t), 1, len(vals) - 1)
    gap = vals[idx] - vals[idx - 1]
    assert np.all(np.abs(t - d) <= gap / 2)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_scale_and_extremes(fmt):
    F = quant.FMAX[fmt]
    g = np.random.default_rng(3)
    x = (g.standard_normal(4097) * 3.7).astype(np.float32)
    q, s = quant.quantize(x, fmt)
    amax = np.float32(np.max(np.abs(x)))
    assert s == np.float32(amax / np.float32(F))
    top = int(np.argmax(np.abs(x)))
    assert abs(decode(q[top:top + 1], fmt)[0]) == F
    # dequantised values are within half a code gap (times s) of x
    t = np.clip(np.float32(x / s), -F, F)
    vals, _ = quant._table(fmt)
    idx = np.clip(np.searchsorted(vals, np.abs(t)), 1, len(vals) - 1)
    assert np.all(np.abs(t - decode(q, fmt)) <= (vals[idx] - vals[idx - 1]) / 2)
    # all-zero tensor
    qz, sz = quant.quantize(np.zeros(33, dtype=np.float32), fmt)
    assert sz == 1.0 and not qz.any()
    # batch form equals per-tensor calls
    qb, sb = quant.quantize_batch(np.concatenate([x, 2 * x]), 4097, 2, fmt)
    q2, s2 = quant.quantize(2 * x, fmt)
    assert np.array_equal(qb[:4097], q) and np.array_equal(qb[4097:], q2)
    assert sb[0] == s and sb[1] == s2


def test_pins_catch_planted_mistakes(monkeypatch):
    """Encoders with a planted mistake fail the torch pin."""
    g = np.random.default_rng(9)
    fmt = "e4m3"
    vals, cs = quant._table(fmt)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([np.clip(g.standard_normal(5000) * 60, -448, 448), mids]).astype(np.float32)

    def ties_away(t, fmt_):
        a = np.abs(t.astype(np.float64))
        hi = np.clip(np.searchsorted(vals, a), 1, len(vals) - 1)
        lo = hi - 1
        pick = (vals[hi] - a) <= (a - vals[lo])
        return (np.where(pick, cs[hi], cs[lo]) | (np.signbit(t).astype(np.uint8) << 7)).astype(np.uint8)

    assert not np.array_equal(ties_away(x, fmt), torch_encode(x, fmt))
    # a scale formed as amax * F instead of amax / F maps the largest element far from F
    xs = (g.standard_normal(100) * 3).astype(np.float32)
    s_bad = np.float32(np.max(np.abs(xs)) * np.float32(448.0))
    t_bad = np.clip(np.float32(xs / s_bad), -448, 448)
    assert np.max(np.abs(decode(quant.encode(t_bad, fmt), fmt))) != 448.0
