"""Pins of the convolution oracle (oracle/conv.py): brute force with plain
loops, reduction to the C oracle's matrix product for 1x1 filters, a delta
filter, shift equivariance, the output-size formula, and planted mistakes."""
import numpy as np
import pytest

from oracle import conv as oc
from oracle import reference


def _brute(x, w, ph, pw, sh, sw, dh, dw):
    N, H, W, C = x.shape
    K, R, S, _ = w.shape
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    y = [[[[0.0] * K for _ in range(Q)] for _ in range(P)] for _ in range(N)]
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                for k in range(K):
                    t = 0.0
                    for r in range(R):
                        for s in range(S):
                            h, ww = p * sh - ph + r * dh, q * sw - pw + s * dw
                            if 0 <= h < H and 0 <= ww < W:
                                for c in range(C):
                                    t += float(x[n, h, ww, c]) * float(w[k, r, s, c])
                    y[n][p][q][k] = t
    return np.array(y)


CASES = [
    # N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw
    (1, 5, 6, 2, 3, 3, 3, 1, 1, 1, 1, 1, 1),
    (2, 7, 5, 3, 2, 3, 2, 2, 0, 2, 1, 1, 2),
    (1, 9, 9, 1, 2, 3, 3, 2, 2, 2, 3, 2, 2),
    (1, 4, 4, 2, 2, 1, 1, 0, 0, 1, 1, 1, 1),
    (1, 3, 8, 2, 1, 2, 5, 0, 3, 1, 2, 1, 1),
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force_small_integers(case):
    N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw = case
    g = np.random.Generator(np.random.PCG64(sum(case)))
    x = g.integers(-3, 4, size=(N, H, W, C)).astype(np.float64)
    w = g.integers(-3, 4, size=(K, R, S, C)).astype(np.float64)
    y, mag = oc.conv2d(x, w, ph, pw, sh, sw, dh, dw)
    ref = _brute(x, w, ph, pw, sh, sw, dh, dw)
    assert y.shape == ref.shape == (N,) + oc.out_size(H, W, R, S, ph, pw, sh, sw, dh, dw) + (K,)
    assert np.array_equal(y, ref)
    assert np.array_equal(mag, _brute(np.abs(x), np.abs(w), ph, pw, sh, sw, dh, dw))
    idx = np.array([[0, 0, 0, 0], [N - 1, y.shape[1] - 1, y.shape[2] - 1, K - 1]])
    e, _ = oc.conv2d_entries(x, w, idx, ph, pw, sh, sw, dh, dw)
    assert np.array_equal(e, y[tuple(idx.T)])


def test_one_by_one_is_the_matrix_product():
    """A 1x1 filter with stride 1 and no padding is C = A B with A the
    pixels (N H W x C) and B the filters: the C oracle's product."""
    g = np.random.Generator(np.random.PCG64(3))
    N, H, W, C, K = 2, 5, 7, 16, 9
    x = g.standard_normal((N, H, W, C))
    w = g.standard_normal((K, 1, 1, C))
    to16 = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xb, wb = to16(x), to16(w)
    y, mag = oc.conv2d(xb, wb)
    Cr, Wr = reference.gemm(N * H * W, K, C, xb.reshape(-1), C, wb.reshape(-1), C)
    assert np.all(np.abs(y.reshape(-1, K) - Cr) <= 1e-12 * Wr)


def test_delta_filter_copies_the_input():
    g = np.random.Generator(np.random.PCG64(4))
    N, H, W, C = 2, 6, 5, 4
    x = g.standard_normal((N, H, W, C))
    w = np.zeros((C, 3, 3, C))
    for c in range(C):
        w[c, 1, 1, c] = 1.0
    y, _ = oc.conv2d(x, w, 1, 1)
    assert np.array_equal(y, x)


def test_shift_equivariance():
    """Stride 1, no padding: moving the image one pixel right moves the
    output one pixel right."""
    g = np.random.Generator(np.random.PCG64(5))
    x = g.integers(-3, 4, size=(1, 8, 9, 3)).astype(np.float64)
    w = g.integers(-3, 4, size=(2, 3, 2, 3)).astype(np.float64)
    y, _ = oc.conv2d(x, w)
    xs = np.zeros_like(x)
    xs[:, :, 1:, :] = x[:, :, :-1, :]
    ys, _ = oc.conv2d(xs, w)
    assert np.array_equal(ys[:, :, 1:, :], y[:, :, :-1, :])


def test_output_size_formula():
    assert oc.out_size(56, 56, 3, 3, 1, 1, 1, 1, 1, 1) == (56, 56)
    assert oc.out_size(224, 224, 7, 7, 3, 3, 2, 2, 1, 1) == (112, 112)
    assert oc.out_size(9, 9, 3, 3, 0, 0, 1, 1, 4, 4) == (1, 1)
    with pytest.raises(ValueError):
        oc.conv2d(np.zeros((1, 2, 2, 1)), np.zeros((1, 3, 3, 1)))


@pytest.mark.parametrize("mutant", ["flip", "stride_ignored", "dilation_ignored", "pad_one_side"])
def test_mutants_are_caught(mutant, monkeypatch):
    """Plausible mistakes planted in the oracle fail the brute-force pin."""
    case = (1, 9, 8, 2, 2, 3, 3, 1, 2, 2, 1, 2, 1)
    N, H, W, C, K, R, S, ph, pw, sh, sw, dh, dw = case
    g = np.random.Generator(np.random.PCG64(6))
    x = g.integers(-3, 4, size=(N, H, W, C)).astype(np.float64)
    w = g.integers(-3, 4, size=(K, R, S, C)).astype(np.float64)
    ref = _brute(x, w, ph, pw, sh, sw, dh, dw)
    orig_window, orig_pad = oc._window, oc._padded
    if mutant == "flip":
        monkeypatch.setattr(oc, "_window", lambda xp, r, s, P, Q, sh_, sw_, dh_, dw_:
                            orig_window(xp, R - 1 - r, S - 1 - s, P, Q, sh_, sw_, dh_, dw_))
    elif mutant == "stride_ignored":
        monkeypatch.setattr(oc, "_window", lambda xp, r, s, P, Q, sh_, sw_, dh_, dw_:
                            orig_window(xp, r, s, P, Q, 1, 1, dh_, dw_))
    elif mutant == "dilation_ignored":
        monkeypatch.setattr(oc, "_window", lambda xp, r, s, P, Q, sh_, sw_, dh_, dw_:
                            orig_window(xp, r, s, P, Q, sh_, sw_, 1, 1))
    else:
        def pad_one_side(xv, ph_, pw_):
            xp = orig_pad(xv, ph_, pw_)
            return np.concatenate([xp[:, ph_:], np.zeros_like(xp[:, :ph_])], axis=1)
        monkeypatch.setattr(oc, "_padded", pad_one_side)
    y, _ = oc.conv2d(x, w, ph, pw, sh, sw, dh, dw)
    assert not np.array_equal(y, ref)
