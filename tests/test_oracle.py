"""Pins for the CPU oracle: the product it computes is checked against things
fixed by the pages and by mathematics, never against itself.

* codecs: every bf16 and E4M3 code against torch's CPU casts (a library
  special case) and hand values of the formats' definitions;
* the FLOP count: the multiply-adds the oracle executes equal MNK, so the
  useful work is 2MNK (FLOPs equation, section "Shape the operation" of page
  "10. Tensor Cores, shapes, and tile alignment");
* numpy's binary64 matrix product (BLAS) on inputs decoded by torch;
* identity and permutation matrices, exact;
* small integers against pure-Python integer sums, exact;
* tiny shapes against exact rational sums;
* the transpose identity through the layout flags, split-K (sum of K-slice
  products), alpha scaling, zero padding, and entry-wise agreement.

A mutation test rebuilds the oracle with planted mistakes and checks that
these pins catch each one.
"""
import itertools
import os
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

from dense_tiled_gemm_fp8_amd import inputs

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]  # (a_colmajor, b_rowmajor)


def lib_decode(codes, fmt=None):
    """Decode with torch's CPU casts (independent of the oracle's decoder);
    uint8 codes are E4M3 unless fmt is "e5m2"."""
    codes = np.ascontiguousarray(codes)
    return inputs.codes_to_torch(codes, fmt).to(torch.float64).numpy()


def store(a_log, b_log, a_colmajor, b_rowmajor):
    """Lay out logical A (M x K) and B (K x N) code arrays in the requested
    storage; returns flat arrays and leading dimensions."""
    M, K = a_log.shape
    _, N = b_log.shape
    if a_colmajor:
        A, lda = np.ascontiguousarray(a_log.T), M      # K rows of M
    else:
        A, lda = np.ascontiguousarray(a_log), K
    if b_rowmajor:
        B, ldb = np.ascontiguousarray(b_log), N        # K rows of N
    else:
        B, ldb = np.ascontiguousarray(b_log.T), K      # N rows of K
    return A.reshape(-1), lda, B.reshape(-1), ldb


def rand_codes(gen, shape, fmt):
    x = gen.uniform(-1, 1, size=shape)
    if fmt == "bf16":
        return inputs.to_bf16_codes(x)
    return inputs.to_fp8_codes(x, fmt)[0]


# ---------------------------------------------------------------- codecs

def test_bf16_decode_exhaustive(oracle_lib):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_lib.decode_bf16(codes)
    ref = lib_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # hand values of the format: 1.0, -2.0, smallest subnormal, largest finite
    assert oracle_lib.decode_bf16(np.array([0x3F80]))[0] == 1.0
    assert oracle_lib.decode_bf16(np.array([0xC000]))[0] == -2.0
    assert oracle_lib.decode_bf16(np.array([0x0001]))[0] == 2.0 ** -133
    assert oracle_lib.decode_bf16(np.array([0x7F7F]))[0] == (2 - 2.0 ** -7) * 2.0 ** 127


def test_e4m3_decode_exhaustive(oracle_lib):
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ours = oracle_lib.decode_e4m3(codes)
    ref = lib_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]          # S.1111.111 only
    hand = {0x7E: 448.0, 0xFE: -448.0, 0x38: 1.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x00: 0.0, 0x80: -0.0, 0x40: 2.0}
    for c, v in hand.items():
        assert oracle_lib.decode_e4m3(np.array([c], dtype=np.uint8))[0] == v
    assert np.nanmax(np.abs(ours)) == 448.0


def test_e4m3_quantiser_clamps(oracle_lib):
    # overflow must clamp to +-448, not become NaN
    q, s = inputs.to_e4m3_codes(np.array([1e6, -1e6, 0.5]), scale=1.0)
    assert list(oracle_lib.decode_e4m3(q)) == [448.0, -448.0, 0.5]


# ---------------------------------------------------------------- FLOPs

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (16, 9, 33), (64, 48, 100)])
def test_mac_count_is_mnk(oracle_lib, M, N, K):
    from oracle import bookkeeping as bk
    g = inputs.rng(1)
    a, b = rand_codes(g, (M, K), "bf16"), rand_codes(g, (K, N), "bf16")
    A, lda, B, ldb = store(a, b, False, False)
    _, _, macs = oracle_lib.gemm(M, N, K, A, lda, B, ldb, return_macs=True)
    assert macs == M * N * K
    assert bk.flops(M, N, K) == 2 * macs


# ---------------------------------------------------------------- library special case

@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(37, 53, 129), (64, 64, 64), (5, 200, 311)])
def test_matches_numpy_float64(oracle_lib, fmt, layout, M, N, K):
    g = inputs.rng(hash((fmt, layout, M, N, K)) & 0xFFFF)
    a, b = rand_codes(g, (M, K), fmt), rand_codes(g, (K, N), fmt)
    A, lda, B, ldb = store(a, b, *layout)
    alpha = 0.375
    C, W = oracle_lib.gemm(M, N, K, A, lda, B, ldb, a_colmajor=layout[0],
                           b_rowmajor=layout[1], alpha=alpha)
    ad, bd = lib_decode(a), lib_decode(b)
    ref = alpha * (ad @ bd)
    wref = abs(alpha) * (np.abs(ad) @ np.abs(bd))
    assert np.all(np.abs(C - ref) <= 1e-12 * wref + 1e-300)
    assert np.allclose(W, wref, rtol=1e-12, atol=0)
    assert np.all(np.abs(C) <= W * (1 + 1e-15))


@pytest.mark.parametrize("fa,fb", [("e5m2", "e5m2"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_matches_numpy_float64_e5m2(oracle_lib, fa, fb, layout):
    M, N, K = 33, 47, 150
    g = inputs.rng(hash((fa, fb, layout)) & 0xFFFF)
    a, b = rand_codes(g, (M, K), fa), rand_codes(g, (K, N), fb)
    A, lda, B, ldb = store(a, b, *layout)
    C, W = oracle_lib.gemm(M, N, K, A, lda, B, ldb, a_colmajor=layout[0], b_rowmajor=layout[1],
                           alpha=-0.75, fmt_a=fa, fmt_b=fb)
    ad, bd = lib_decode(a, fa), lib_decode(b, fb)
    ref = -0.75 * (ad @ bd)
    wref = 0.75 * (np.abs(ad) @ np.abs(bd))
    assert np.all(np.abs(C - ref) <= 1e-12 * wref + 1e-300)
    assert np.allclose(W, wref, rtol=1e-12, atol=0)
    c, w = oracle_lib.gemm_entries(K, A, lda, B, ldb, np.arange(M), np.arange(M) % N, *layout, alpha=-0.75,
                                   fmt_a=fa, fmt_b=fb)
    assert np.array_equal(c, C[np.arange(M), np.arange(M) % N])


def test_entries_equal_full(oracle_lib):
    M, N, K = 70, 90, 257
    g = inputs.rng(7)
    a, b = rand_codes(g, (M, K), "bf16"), rand_codes(g, (K, N), "bf16")
    for layout in LAYOUTS:
        A, lda, B, ldb = store(a, b, *layout)
        C, W = oracle_lib.gemm(M, N, K, A, lda, B, ldb, *layout, alpha=1.5)
        ii = g.integers(0, M, 300)
        jj = g.integers(0, N, 300)
        c, w = oracle_lib.gemm_entries(K, A, lda, B, ldb, ii, jj, *layout, alpha=1.5)
        assert np.array_equal(c, C[ii, jj])
        assert np.array_equal(w, W[ii, jj])


# ---------------------------------------------------------------- exact structure

@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_identity_and_permutation(oracle_lib, fmt, layout):
    M, K = 23, 40
    g = inputs.rng(11)
    a = rand_codes(g, (M, K), fmt)
    one = inputs.to_bf16_codes(np.eye(K)) if fmt == "bf16" else inputs.to_e4m3_codes(np.eye(K), 1.0)[0]
    A, lda, B, ldb = store(a, one, *layout)
    C, _ = oracle_lib.gemm(M, K, K, A, lda, B, ldb, *layout)
    assert np.array_equal(C, lib_decode(a))
    perm = g.permutation(K)
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0                       # column j of A.P is column perm[j] of A
    pc = inputs.to_bf16_codes(P) if fmt == "bf16" else inputs.to_e4m3_codes(P, 1.0)[0]
    A, lda, B, ldb = store(a, pc, *layout)
    C, _ = oracle_lib.gemm(M, K, K, A, lda, B, ldb, *layout)
    assert np.array_equal(C, lib_decode(a)[:, perm])


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_small_integers_exact(oracle_lib, fmt):
    g = inputs.rng(5)
    for (M, N, K) in [(1, 1, 1), (7, 3, 19), (16, 16, 16), (9, 31, 64)]:
        a = inputs.small_int_codes(g, (M, K), fmt)
        b = inputs.small_int_codes(g, (K, N), fmt)
        ai = lib_decode(a).astype(int).tolist()
        bi = lib_decode(b).astype(int).tolist()
        want = [[sum(ai[i][k] * bi[k][j] for k in range(K)) for j in range(N)] for i in range(M)]
        for layout in LAYOUTS:
            A, lda, B, ldb = store(a, b, *layout)
            C, W = oracle_lib.gemm(M, N, K, A, lda, B, ldb, *layout)
            assert C.tolist() == [[float(v) for v in row] for row in want]
            wabs = [[sum(abs(ai[i][k] * bi[k][j]) for k in range(K)) for j in range(N)] for i in range(M)]
            assert W.tolist() == [[float(v) for v in row] for row in wabs]


def _exact_value(code, fmt):
    """Decode one code to a Fraction from the format definition."""
    code = int(code)
    if fmt == "bf16":
        s, e, m = code >> 15, (code >> 7) & 0xFF, code & 0x7F
        mag = Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    else:
        s, e, m = code >> 7, (code >> 3) & 0xF, code & 0x7
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_tiny_shapes_brute_force(oracle_lib, fmt):
    dims = [1, 2, 3, 7, 8, 15, 16]
    g = inputs.rng(3 if fmt == "bf16" else 4)
    for M, N, K in itertools.product(dims, dims, dims):
        a, b = rand_codes(g, (M, K), fmt), rand_codes(g, (K, N), fmt)
        fa = [[_exact_value(a[i, k], fmt) for k in range(K)] for i in range(M)]
        fb = [[_exact_value(b[k, j], fmt) for j in range(N)] for k in range(K)]
        A, lda, B, ldb = store(a, b, False, False)
        C, W = oracle_lib.gemm(M, N, K, A, lda, B, ldb)
        for i in range(M):
            for j in range(N):
                exact = sum((fa[i][k] * fb[k][j] for k in range(K)), Fraction(0))
                wexact = sum((abs(fa[i][k] * fb[k][j]) for k in range(K)), Fraction(0))
                # binary64 sums of exact products: error at most K * 2^-53 * W
                assert abs(Fraction(C[i, j]) - exact) <= K * Fraction(1, 2 ** 53) * wexact
                assert abs(Fraction(W[i, j]) - wexact) <= K * Fraction(1, 2 ** 53) * wexact


# ---------------------------------------------------------------- invariants

def test_transpose_identity(oracle_lib):
    """(A B)^T = B^T A^T: the same buffers, read through swapped layout flags."""
    M, N, K = 33, 21, 77
    g = inputs.rng(9)
    a, b = rand_codes(g, (M, K), "bf16"), rand_codes(g, (K, N), "bf16")
    for layout in LAYOUTS:
        A, lda, B, ldb = store(a, b, *layout)
        C, _ = oracle_lib.gemm(M, N, K, A, lda, B, ldb, *layout)
        # B^T is N x K: row-major iff B was column-major; A^T is K x M:
        # column-major iff A was row-major.
        Ct, _ = oracle_lib.gemm(N, M, K, B, ldb, A, lda, a_colmajor=layout[1],
                                b_rowmajor=layout[0])
        assert np.array_equal(Ct, C.T)


def test_split_k_sum(oracle_lib):
    """Sum over K-slices of slice products equals the full product: exact for
    small integers, within the binary64 bound for floats."""
    from oracle import bookkeeping as bk
    M, N, K = 19, 26, 300
    g = inputs.rng(13)
    for ints in (True, False):
        if ints:
            a, b = inputs.small_int_codes(g, (M, K), "bf16"), inputs.small_int_codes(g, (K, N), "bf16")
        else:
            a, b = rand_codes(g, (M, K), "bf16"), rand_codes(g, (K, N), "bf16")
        full, W = oracle_lib.gemm(M, N, K, np.ascontiguousarray(a).reshape(-1), K,
                                  np.ascontiguousarray(b.T).reshape(-1), K)
        for s in (2, 3, 7, 300):
            acc = np.zeros((M, N))
            for (kb, ke) in bk.kslices(K, s):
                if ke == kb:
                    continue
                part, _ = oracle_lib.gemm(M, N, ke - kb,
                                          np.ascontiguousarray(a[:, kb:ke]).reshape(-1), ke - kb,
                                          np.ascontiguousarray(b[kb:ke, :].T).reshape(-1), ke - kb)
                acc += part
            if ints:
                assert np.array_equal(acc, full)
            else:
                assert np.all(np.abs(acc - full) <= 2 * K * 2.0 ** -53 * W)


def test_alpha_scaling(oracle_lib):
    M, N, K = 12, 14, 50
    g = inputs.rng(17)
    a, b = rand_codes(g, (M, K), "e4m3"), rand_codes(g, (K, N), "e4m3")
    A, lda, B, ldb = store(a, b, False, False)
    C1, W1 = oracle_lib.gemm(M, N, K, A, lda, B, ldb)
    for alpha in (0.25, -8.0, 2.0 ** -20):
        Ca, Wa = oracle_lib.gemm(M, N, K, A, lda, B, ldb, alpha=alpha)
        assert np.array_equal(Ca, alpha * C1)
        assert np.array_equal(Wa, abs(alpha) * W1)


def test_zero_padding(oracle_lib):
    M, N, K = 29, 35, 61
    Mp, Np, Kp = 64, 64, 128
    g = inputs.rng(19)
    a, b = rand_codes(g, (M, K), "bf16"), rand_codes(g, (K, N), "bf16")
    ap = np.zeros((Mp, Kp), dtype=np.uint16)
    bp = np.zeros((Kp, Np), dtype=np.uint16)
    ap[:M, :K] = a
    bp[:K, :N] = b
    A, lda, B, ldb = store(a, b, False, False)
    C, W = oracle_lib.gemm(M, N, K, A, lda, B, ldb)
    A, lda, B, ldb = store(ap, bp, False, False)
    Cp, Wp = oracle_lib.gemm(Mp, Np, Kp, A, lda, B, ldb)
    assert np.array_equal(Cp[:M, :N], C)
    assert not Cp[M:, :].any() and not Cp[:, N:].any()


def test_leading_dimension_padding(oracle_lib):
    """Leading dimensions larger than the logical extent address the same
    logical matrices."""
    M, N, K = 17, 13, 40
    g = inputs.rng(23)
    a, b = rand_codes(g, (M, K), "bf16"), rand_codes(g, (K, N), "bf16")
    A, lda, B, ldb = store(a, b, False, False)
    C, _ = oracle_lib.gemm(M, N, K, A, lda, B, ldb)
    Aw = np.full((M, K + 9), 0x7FC0, dtype=np.uint16)       # NaN filler never read
    Aw[:, :K] = a
    Bw = np.full((N, K + 5), 0x7FC0, dtype=np.uint16)
    Bw[:, :K] = b.T
    C2, _ = oracle_lib.gemm(M, N, K, Aw.reshape(-1), K + 9, Bw.reshape(-1), K + 5)
    assert np.array_equal(C, C2)


# ---------------------------------------------------------------- pins catch planted mistakes

MUTANTS = {
    "dropped_last_term": ("for (k = 0; k < K; ++k) {\n            const double aik", "for (k = 0; k < K - 1; ++k) {\n            const double aik"),
    "wrong_sign": ("c[j] += p;", "c[j] -= p;"),
    "transposed_a": ("return a_colmajor ? k * lda + i : i * lda + k;", "return a_colmajor ? i * lda + k : k * lda + i;"),
    "transposed_b": ("return b_rowmajor ? k * ldb + j : j * ldb + k;", "return b_rowmajor ? j * ldb + k : k * ldb + j;"),
    "e4m3_bias": ("ldexp(8.0 + (double)m, e - 10)", "ldexp(8.0 + (double)m, e - 11)"),
    "e4m3_subnormal": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e5m2_bias": ("ldexp(4.0 + (double)m, e - 17)", "ldexp(4.0 + (double)m, e - 16)"),
    "e5m2_subnormal": ("ldexp((double)m, -16)", "ldexp((double)m, -15)"),
    "b_format_ignored": ("b[k * N + j] = decode(B, b_index(k, j, ldb, b_rowmajor), fmt_b);",
                         "b[k * N + j] = decode(B, b_index(k, j, ldb, b_rowmajor), fmt_a);"),
    "no_alpha": ("c[j] *= alpha;", "c[j] *= 1.0;"),
}


def _pins_pass(lib_path):
    """A compact run of the numpy, identity and codec pins against an oracle
    library at ``lib_path``; returns False on the first failure."""
    import ctypes
    from oracle import reference as r
    saved = r._lib
    try:
        r._lib = None
        old = r._LIB_PATH
        r._LIB_PATH = lib_path
        try:
            lib = r._load()
        finally:
            r._LIB_PATH = old
        codes8 = np.arange(256, dtype=np.uint16).astype(np.uint8)
        ref8 = lib_decode(codes8)
        got8 = r.decode_e4m3(codes8)
        ok = np.array_equal(np.nan_to_num(got8, nan=7.0), np.nan_to_num(ref8, nan=7.0))
        ref5 = lib_decode(codes8, "e5m2")
        got5 = r.decode_e5m2(codes8)
        ok &= np.array_equal(np.nan_to_num(got5, nan=7.0), np.nan_to_num(ref5, nan=7.0))
        g = inputs.rng(29)
        for fa, fb in (("bf16", "bf16"), ("e4m3", "e4m3"), ("e4m3", "e5m2")):
            M, N, K = 9, 11, 37
            a, b = rand_codes(g, (M, K), fa), rand_codes(g, (K, N), fb)
            ad, bd = lib_decode(a, fa), lib_decode(b, fb)
            for layout in LAYOUTS:
                A, lda, B, ldb = store(a, b, *layout)
                C, W = r.gemm(M, N, K, A, lda, B, ldb, *layout, alpha=0.5,
                              fmt_a=None if fa == "bf16" else fa, fmt_b=None if fb == "bf16" else fb)
                ref = 0.5 * (ad @ bd)
                wref = 0.5 * (np.abs(ad) @ np.abs(bd))
                ok &= bool(np.all(np.abs(C - ref) <= 1e-12 * wref))
        return bool(ok)
    finally:
        r._lib = saved


def test_pins_catch_planted_mistakes(oracle_lib):
    src = open(oracle_lib._SRC).read()
    assert _pins_pass(oracle_lib._LIB_PATH)
    with tempfile.TemporaryDirectory() as d:
        for name, (old, new) in MUTANTS.items():
            assert old in src, name
            path = os.path.join(d, name + ".c")
            with open(path, "w") as f:
                f.write(src.replace(old, new))
            so = os.path.join(d, name + ".so")
            subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                            path, "-o", so, "-lm"], check=True)
            assert not _pins_pass(so), "pin suite missed mutant %s" % name
