"""Pins of the block-scaled product oracle (oracle/mx.py) against things
outside it: torch's E8M0 type, closed forms, and the plain binary64 product
of gemm_oracle.c applied block by block.

The pages name microscaling only as a row of the precision table on page
"The Tensor Core"; the format definition followed is the OCP Microscaling
Formats specification v1.0 (32-element blocks along K, E8M0 scales).
"""
import numpy as np
import pytest
import torch

from oracle import mx
from oracle import reference

E4M3_ONE = 0x38      # 1.0 in E4M3: exponent field 7 (bias 7), mantissa 0
E5M2_ONE = 0x3C      # 1.0 in E5M2: exponent field 15 (bias 15), mantissa 0


def _codes(gen, shape, fmt):
    """Random finite codes of the format."""
    c = gen.integers(0, 256, size=shape).astype(np.uint8)
    if fmt == "e4m3":
        c[(c & 0x7F) == 0x7F] = 0x10
    else:
        c[(c & 0x7C) == 0x7C] = 0x10
    return c


def test_e8m0_matches_torch():
    """Every E8M0 code decodes as torch's float8_e8m0fnu does."""
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mx.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_element_decoders_are_the_pinned_ones():
    assert mx._element_table("e4m3")[E4M3_ONE] == 1.0
    assert mx._element_table("e5m2")[E5M2_ONE] == 1.0
    with pytest.raises(ValueError):
        mx._element_table("bf16")


@pytest.mark.parametrize("fmt,one", [("e4m3", E4M3_ONE), ("e5m2", E5M2_ONE)])
def test_all_ones_closed_form(fmt, one):
    """A and B all 1.0: C[i][j] = sum over blocks of (block length) *
    2^(sa[i][b] + sb[j][b] - 254), the last block holding K mod 32
    elements."""
    g = np.random.Generator(np.random.PCG64(5))
    M, N, K = 7, 5, 100                     # 4 blocks, the last of 4 elements
    nb = 4
    sa = g.integers(110, 140, size=(M, nb)).astype(np.uint8)
    sb = g.integers(110, 140, size=(N, nb)).astype(np.uint8)
    A = np.full((M, K), one, dtype=np.uint8)
    B = np.full((N, K), one, dtype=np.uint8)
    C, W = mx.gemm(A, sa, B, sb, fmt)
    lens = np.array([32, 32, 32, 4], dtype=np.float64)
    want = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            want[i, j] = sum(lens[b] * 2.0 ** (int(sa[i, b]) + int(sb[j, b]) - 254) for b in range(nb))
    assert np.array_equal(C, want)
    assert np.array_equal(W, want)


@pytest.mark.parametrize("fmt_a,fmt_b", [("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2")])
def test_unit_scales_reduce_to_plain_product(fmt_a, fmt_b):
    """With every scale 127 (2^0) the block-scaled product is the plain
    product of the C oracle."""
    g = np.random.Generator(np.random.PCG64(6))
    M, N, K = 33, 17, 96
    A, B = _codes(g, (M, K), fmt_a), _codes(g, (N, K), fmt_b)
    ones_a = np.full((M, 3), 127, dtype=np.uint8)
    ones_b = np.full((N, 3), 127, dtype=np.uint8)
    C, W = mx.gemm(A, ones_a, B, ones_b, fmt_a, fmt_b, alpha=0.75)
    Cr, Wr = reference.gemm(M, N, K, A.reshape(-1), K, B.reshape(-1), K, alpha=0.75, fmt_a=fmt_a, fmt_b=fmt_b)
    assert np.all(np.abs(C - Cr) <= 1e-12 * Wr)
    assert np.all(np.abs(W - Wr) <= 1e-12 * Wr)


def _blockwise(A, sa, B, sb, fmt_a, fmt_b):
    """The product as a sum over K-blocks of the C oracle's plain product of
    the block, times the two scales of the block."""
    M, K = A.shape
    N = B.shape[0]
    C = np.zeros((M, N))
    W = np.zeros((M, N))
    for b in range(-(-K // 32)):
        k0, k1 = 32 * b, min(K, 32 * b + 32)
        Ab = np.ascontiguousarray(A[:, k0:k1])
        Bb = np.ascontiguousarray(B[:, k0:k1])
        Cb, Wb = reference.gemm(M, N, k1 - k0, Ab.reshape(-1), k1 - k0, Bb.reshape(-1), k1 - k0,
                                fmt_a=fmt_a, fmt_b=fmt_b)
        f = np.ldexp(1.0, sa[:, b].astype(np.int64)[:, None] + sb[:, b].astype(np.int64)[None, :] - 254)
        C += f * Cb
        W += f * Wb
    return C, W


@pytest.mark.parametrize("fmt_a,fmt_b,K", [("e4m3", "e4m3", 256), ("e5m2", "e5m2", 160),
                                            ("e4m3", "e5m2", 70)])
def test_block_decomposition(fmt_a, fmt_b, K):
    """Random scales: the product equals the block-by-block sum of plain
    products scaled by 2^(sa + sb - 254); a scale attached to the wrong row,
    column or block breaks it."""
    g = np.random.Generator(np.random.PCG64(7))
    M, N = 19, 23
    nb = -(-K // 32)
    A, B = _codes(g, (M, K), fmt_a), _codes(g, (N, K), fmt_b)
    sa = g.integers(100, 150, size=(M, nb)).astype(np.uint8)
    sb = g.integers(100, 150, size=(N, nb)).astype(np.uint8)
    C, W = mx.gemm(A, sa, B, sb, fmt_a, fmt_b)
    Cr, Wr = _blockwise(A, sa, B, sb, fmt_a, fmt_b)
    assert np.all(np.abs(C - Cr) <= 1e-12 * Wr)
    assert np.all(np.abs(W - Wr) <= 1e-12 * Wr)
    rows = np.array([0, 5, M - 1, 3]), np.array([N - 1, 2, 0, 22])
    c, w = mx.gemm_entries(A, sa, B, sb, rows[0], rows[1], fmt_a, fmt_b)
    assert np.all(np.abs(c - Cr[rows]) <= 1e-12 * Wr[rows])


def test_nan_scale_gives_nan():
    A = np.full((2, 64), E4M3_ONE, dtype=np.uint8)
    B = np.full((2, 64), E4M3_ONE, dtype=np.uint8)
    sa = np.full((2, 2), 127, dtype=np.uint8)
    sb = np.full((2, 2), 127, dtype=np.uint8)
    sa[1, 1] = 255
    C, _ = mx.gemm(A, sa, B, sb)
    assert not np.isnan(C[0]).any() and np.isnan(C[1]).all()


def test_shape_checks():
    A = np.zeros((4, 64), dtype=np.uint8)
    with pytest.raises(ValueError):
        mx.scaled_operand(A, np.zeros((4, 3), dtype=np.uint8), "e4m3")


@pytest.mark.parametrize("mutant", ["block16", "no_bias", "scales_swapped"])
def test_mutants_are_caught(mutant, monkeypatch):
    """Plausible mistakes in the oracle fail the decomposition pin."""
    g = np.random.Generator(np.random.PCG64(8))
    M, N, K = 8, 8, 128
    A, B = _codes(g, (M, K), "e4m3"), _codes(g, (N, K), "e4m3")
    sa = g.integers(110, 140, size=(M, 4)).astype(np.uint8)
    sb = g.integers(110, 140, size=(N, 4)).astype(np.uint8)
    Cr, Wr = _blockwise(A, sa, B, sb, "e4m3", "e4m3")
    if mutant == "block16":
        orig = mx.scaled_operand

        def scaled16(codes, scales, fmt):
            vals = mx._element_table(fmt)[np.asarray(codes, dtype=np.uint8)]
            per_k = np.repeat(mx.decode_e8m0(scales), 16, axis=1)
            per_k = np.concatenate([per_k, per_k], axis=1)[:, :codes.shape[1]]
            return vals * per_k
        monkeypatch.setattr(mx, "scaled_operand", scaled16)
        C, _ = mx.gemm(A, sa, B, sb)
        monkeypatch.setattr(mx, "scaled_operand", orig)
    elif mutant == "no_bias":
        monkeypatch.setattr(mx, "decode_e8m0", lambda c: np.ldexp(1.0, np.asarray(c, dtype=np.int64) - 120))
        C, _ = mx.gemm(A, sa, B, sb)
    else:
        C, _ = mx.gemm(A, sb, B, sa)
    assert not np.all(np.abs(C - Cr) <= 1e-6 * Wr)


def test_e2m1_decoder_matches_spec_table():
    """Every FP4 E2M1 code against the value table of the OCP MX
    specification (tests/golden/e2m1_values.json)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.json")
    table = json.load(open(path))["values"]
    got = mx.decode_e2m1(np.arange(16))
    for code, v in table.items():
        assert got[int(code)] == v and np.signbit(got[int(code)]) == np.signbit(v), code
    # the high nibble is ignored by the decoder; packing puts element 2i low
    assert np.array_equal(mx.unpack_fp4(np.array([[0x72, 0x1F]], dtype=np.uint8)),
                          np.array([[2, 7, 15, 1]], dtype=np.uint8))


def test_e2m1_input_rounding_is_nearest_even():
    """The input generator's E2M1 rounding (inputs.to_e2m1_codes): nearest
    value of the oracle's table, ties to the even code, saturation at 6."""
    from dense_tiled_gemm_fp8_amd import inputs
    vals = mx.decode_e2m1(np.arange(8))
    g = np.random.Generator(np.random.PCG64(9))
    y = np.concatenate([g.uniform(-7, 7, 4000), (vals[1:] + vals[:-1]) / 2, -(vals[1:] + vals[:-1]) / 2, vals])
    c = inputs.to_e2m1_codes(y)
    dec = mx.decode_e2m1(c)
    mag = np.minimum(np.abs(y), 6.0)
    err = np.abs(np.abs(dec) - mag)
    best = np.min(np.abs(vals[None, :] - mag[:, None]), axis=1)
    assert np.all(err == best)
    tie = np.isclose(np.abs(vals[None, :] - mag[:, None]), best[:, None], rtol=0, atol=0).sum(axis=1) > 1
    assert np.all((c[tie] & 1) == 0)
    assert np.all(np.signbit(dec[y != 0]) == np.signbit(y[y != 0]))


def test_fp4_all_ones_closed_form():
    """FP4 1.0 is code 2; packed all-ones operands give the closed form."""
    g = np.random.Generator(np.random.PCG64(10))
    M, N, K = 5, 6, 256
    sa = g.integers(115, 135, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(115, 135, size=(N, K // 32)).astype(np.uint8)
    A = np.full((M, K // 2), 0x22, dtype=np.uint8)
    B = np.full((N, K // 2), 0x22, dtype=np.uint8)
    C, _ = mx.gemm(A, sa, B, sb, "e2m1")
    want = np.array([[sum(32 * 2.0 ** (int(sa[i, b]) + int(sb[j, b]) - 254) for b in range(K // 32))
                      for j in range(N)] for i in range(M)])
    assert np.array_equal(C, want)


def test_fp4_block_decomposition_through_e4m3():
    """Every E2M1 value is an E4M3 value: the FP4 product equals the 8-bit
    product of the same values re-encoded as E4M3 by torch's cast, through
    the C oracle, block by block."""
    g = np.random.Generator(np.random.PCG64(11))
    M, N, K = 9, 7, 256
    A4 = g.integers(0, 256, size=(M, K // 2)).astype(np.uint8)
    B4 = g.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    sa = g.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    C4, W4 = mx.gemm(A4, sa, B4, sb, "e2m1")
    to8 = lambda p: torch.from_numpy(mx.decode_e2m1(mx.unpack_fp4(p)).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    Cr, Wr = _blockwise(to8(A4), sa, to8(B4), sb, "e4m3", "e4m3")
    assert np.all(np.abs(C4 - Cr) <= 1e-12 * Wr)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_decoders_match_spec_values(fmt):
    """Every 6-bit code against the magnitudes of the OCP specification's
    format parameters (tests/golden/fp6_values.json: bias, mantissa width
    and the listed extremes), sign in bit 5."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "fp6_values.json")
    table = json.load(open(path))[fmt]
    dec = mx.decode_e2m3 if fmt == "e2m3" else mx.decode_e3m2
    got = dec(np.arange(64))
    for code, v in table.items():
        assert got[int(code)] == v
        assert got[int(code) | 32] == -v and np.signbit(got[int(code) | 32])
    assert np.all(np.diff(got[:32]) > 0)


def test_fp6_bit_stream_order():
    """Element i sits in bits 6i .. 6i+5 of its row (little-endian)."""
    packed = np.array([[0b11000001, 0b00000000, 0b00000000]], dtype=np.uint8)   # e0 = 1, e1 = 3
    assert mx.unpack_fp6(packed).tolist() == [[1, 3, 0, 0]]
    packed = np.array([[0, 0, 0b11111100]], dtype=np.uint8)                     # e3 = 63
    assert mx.unpack_fp6(packed).tolist() == [[0, 0, 0, 63]]


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_product_through_e4m3(fmt):
    """Every E2M3 and E3M2 value is an E4M3 value: the FP6 product equals
    the 8-bit product of the same values re-encoded as E4M3 by torch's cast,
    block by block through the C oracle."""
    from dense_tiled_gemm_fp8_amd import inputs
    g = np.random.Generator(np.random.PCG64(13))
    M, N, K = 9, 7, 256
    A6 = inputs.pack_fp6(g.integers(0, 64, size=(M, K)).astype(np.uint8))
    B6 = inputs.pack_fp6(g.integers(0, 64, size=(N, K)).astype(np.uint8))
    sa = g.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    sb = g.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    C6, _ = mx.gemm(A6, sa, B6, sb, fmt)
    dec = mx.decode_e2m3 if fmt == "e2m3" else mx.decode_e3m2
    to8 = lambda p: torch.from_numpy(dec(mx.unpack_fp6(p)).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    Cr, Wr = _blockwise(to8(A6), sa, to8(B6), sb, "e4m3", "e4m3")
    assert np.all(np.abs(C6 - Cr) <= 1e-12 * Wr)


def test_fp6_input_rounding_is_nearest_even():
    from dense_tiled_gemm_fp8_amd import inputs
    for fmt, dec in (("e2m3", mx.decode_e2m3), ("e3m2", mx.decode_e3m2)):
        vals = dec(np.arange(32))
        g = np.random.Generator(np.random.PCG64(14))
        y = np.concatenate([g.uniform(-40, 40, 3000), (vals[1:] + vals[:-1]) / 2, vals])
        c = inputs.to_fp6_codes(y, fmt)
        mag = np.minimum(np.abs(y), vals[-1])
        best = np.min(np.abs(vals[None, :] - mag[:, None]), axis=1)
        assert np.all(np.abs(np.abs(dec(c)) - mag) == best)
        tie = (np.abs(vals[None, :] - mag[:, None]) == best[:, None]).sum(axis=1) > 1
        assert np.all((c[tie] & 1) == 0)
