"""Pins of the oracle's depthwise 3x3 inner model (no GPU).

The conv head is checked against torch's own depthwise conv2d (a library
routine: cross-correlation, zero padding), a brute-force im2col
least-squares gradient, central finite differences of the loss, and closed
forms (reconstructible values give g = 0; a delta kernel reproduces its
input).  Non-square grids catch a transposed (y, x) reading of the tokens.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _rand(rng, B, H, gh, gw, d):
    N = gh * gw
    K = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    Q = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    V = rng.standard_normal((B, H, N, d))
    w0 = rng.standard_normal((H, d, 3, 3)) / 3.0
    eta = rng.uniform(0.5, 2.0, size=H)
    return K, Q, V, w0, eta


def _conv(X, w, gh, gw):
    """Depthwise conv of one [N,d] token map with w [d,3,3] via torch."""
    d = X.shape[-1]
    img = torch.from_numpy(X.reshape(gh, gw, d).transpose(2, 0, 1).copy())[None]
    out = F.conv2d(img, torch.from_numpy(w.copy())[:, None], padding=1, groups=d)
    return out[0].numpy().transpose(1, 2, 0).reshape(gh * gw, d)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_reconstructible_values_give_zero_gradient():
    rng = np.random.default_rng(20)
    gh, gw, d = 6, 9, 8
    K, Q, _, w0, eta = _rand(rng, 2, 1, gh, gw, d)
    V = np.stack([_conv(K[b, 0], w0[0], gh, gw) for b in range(2)])[:, None]
    _, g = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    assert np.max(np.abs(g)) < 1e-14


def test_delta_kernel_reproduces_input():
    rng = np.random.default_rng(21)
    gh, gw, d = 5, 7, 4
    K, Q, V, w0, eta = _rand(rng, 1, 1, gh, gw, d)
    w0[:] = 0.0
    w0[:, :, 1, 1] = 1.0
    eta[:] = 0.0
    Z, g = oracle.dwconv3x3_fullbatch(K, Q, V.copy(), w0, eta, gh, gw)
    assert _rel(Z, Q) < 1e-15
    # P = K when w0 is the delta, so with V = K the update is zero.
    _, g2 = oracle.dwconv3x3_fullbatch(K, Q, K.copy(), w0, np.ones(1), gh, gw)
    assert np.max(np.abs(g2)) < 1e-15


def test_gradient_matches_im2col_least_squares():
    # Per channel: X[n, tap] = K shifted by the tap, loss (1/N)||X w - v||^2,
    # gradient (2/N) X^T (X w - v).
    rng = np.random.default_rng(22)
    gh, gw, d = 7, 5, 6
    K, Q, V, w0, eta = _rand(rng, 1, 2, gh, gw, d)
    _, g = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    N = gh * gw
    for h in range(2):
        for c in range(d):
            img = np.pad(K[0, h, :, c].reshape(gh, gw), 1)
            X = np.zeros((N, 9))
            for i in range(3):
                for j in range(3):
                    X[:, 3 * i + j] = img[i:i + gh, j:j + gw].reshape(-1)
            w = w0[h, c].reshape(9)
            ref = (2.0 / N) * X.T @ (X @ w - V[0, h, :, c])
            assert _rel(g[0, h, c].reshape(9), ref) < 1e-12


def test_gradient_matches_finite_differences():
    rng = np.random.default_rng(23)
    gh, gw, d = 4, 6, 3
    K, Q, V, w0, eta = _rand(rng, 1, 1, gh, gw, d)
    _, g = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    N = gh * gw

    def loss(w):
        P = _conv(K[0, 0], w, gh, gw)
        return np.sum((P - V[0, 0]) ** 2) / N

    h = 1e-6
    for c in range(d):
        for t in range(9):
            wp = w0[0].copy(); wp[c].reshape(-1)[t] += h
            wm = w0[0].copy(); wm[c].reshape(-1)[t] -= h
            fd = (loss(wp) - loss(wm)) / (2 * h)
            assert abs(fd - g[0, 0, c].reshape(-1)[t]) < 1e-7 * max(1.0, abs(fd))


def test_output_is_conv_with_updated_kernel():
    rng = np.random.default_rng(24)
    gh, gw, d = 9, 4, 8
    K, Q, V, w0, eta = _rand(rng, 2, 2, gh, gw, d)
    Z, g = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    for b in range(2):
        for h in range(2):
            w1 = w0[h] - eta[h] * g[b, h]
            assert _rel(Z[b, h], _conv(Q[b, h], w1, gh, gw)) < 1e-13


def test_single_pixel_grid():
    # 1x1 grid: only the centre tap sees data.
    rng = np.random.default_rng(25)
    K, Q, V, w0, eta = _rand(rng, 1, 1, 1, 1, 4)
    Z, g = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, 1, 1)
    gc = 2.0 * (w0[0, :, 1, 1] * K[0, 0, 0] - V[0, 0, 0]) * K[0, 0, 0]
    assert _rel(g[0, 0, :, 1, 1], gc) < 1e-14
    mask = np.ones((3, 3), bool); mask[1, 1] = False
    assert np.all(g[0, 0][:, mask] == 0.0)
    assert _rel(Z[0, 0, 0], (w0[0, :, 1, 1] - eta[0] * gc) * Q[0, 0, 0]) < 1e-14
