"""Pins of the oracle's backward of the depthwise 3x3 full-batch step (no GPU).

The reverse-mode loops of ``oracle.dwconv3x3_fullbatch_bwd`` are checked
against things they share no code with:
  * central finite differences of L = <dZ, Z> through the (separately
    pinned) forward oracle, for every entry of K, Q, V, w0 and eta;
  * the same gradients derived independently in matrix form per channel
    (im2col: X_K w0 = P, g = (2/N) X_K^T (X_K w0 - v), z = X_Q w1), with
    the column-to-image scatter done by numpy index arithmetic;
  * torch's conv_transpose2d (a library routine, the adjoint of conv2d)
    for dQ;
  * closed forms: eta = 0 gives dK = dV = 0; dW0 and deta are sums over the
    batch of the per-image results; dV is non-zero through the update.
Non-square grids catch a transposed (y, x) reading.
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
    dZ = rng.standard_normal((B, H, N, d))
    return K, Q, V, w0, eta, dZ


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _loss(K, Q, V, w0, eta, dZ, gh, gw):
    Z, _ = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    return float(np.sum(dZ * Z))


def test_finite_differences_of_every_input():
    rng = np.random.default_rng(40)
    B, H, gh, gw, d = 2, 2, 4, 5, 3
    K, Q, V, w0, eta, dZ = _rand(rng, B, H, gh, gw, d)
    dK, dQ, dV, dw0, deta = oracle.dwconv3x3_fullbatch_bwd(K, Q, V, w0, eta, dZ, gh, gw)
    args = [K, Q, V, w0, eta]
    grads = [dK, dQ, dV, dw0, deta]
    h = 1e-6
    for a, gr in zip(args, grads):
        fd = np.empty_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = a[ix]
            a[ix] = old + h
            lp = _loss(*args, dZ, gh, gw)
            a[ix] = old - h
            lm = _loss(*args, dZ, gh, gw)
            a[ix] = old
            fd[ix] = (lp - lm) / (2 * h)
        assert _rel(gr, fd) < 1e-7, (_rel(gr, fd), a.shape)


def _im2col(X, gh, gw):
    """[N] channel map -> [N, 9] zero-padded 3x3 windows (tap t = 3 i + j)."""
    img = np.zeros((gh + 2, gw + 2))
    img[1:-1, 1:-1] = X.reshape(gh, gw)
    cols = np.empty((gh * gw, 9))
    for i in range(3):
        for j in range(3):
            cols[:, 3 * i + j] = img[i:i + gh, j:j + gw].reshape(-1)
    return cols


def _col2im(C, gh, gw):
    """Adjoint of _im2col: scatter-add the 9 window columns back to pixels."""
    img = np.zeros((gh + 2, gw + 2))
    for i in range(3):
        for j in range(3):
            img[i:i + gh, j:j + gw] += C[:, 3 * i + j].reshape(gh, gw)
    return img[1:-1, 1:-1].reshape(-1)


def _matrix_form(K, Q, V, w0, eta, dZ, gh, gw):
    B, H, N, d = K.shape
    dK, dQ, dV = np.zeros_like(K), np.zeros_like(K), np.zeros_like(K)
    dw0 = np.zeros((H, d, 3, 3))
    deta = np.zeros(H)
    for b in range(B):
        for h in range(H):
            for c in range(d):
                w = w0[h, c].reshape(9)
                XK, XQ = _im2col(K[b, h, :, c], gh, gw), _im2col(Q[b, h, :, c], gh, gw)
                v, dz = V[b, h, :, c], dZ[b, h, :, c]
                R = XK @ w - v
                g = (2.0 / N) * XK.T @ R
                w1 = w - eta[h] * g
                dw1 = XQ.T @ dz
                dQ[b, h, :, c] = _col2im(np.outer(dz, w1), gh, gw)
                dg = -eta[h] * dw1
                deta[h] += -dw1 @ g
                dR = (2.0 / N) * XK @ dg
                dV[b, h, :, c] = -dR
                dK[b, h, :, c] = _col2im((2.0 / N) * np.outer(R, dg) + np.outer(dR, w), gh, gw)
                dw0[h, c] += (dw1 + XK.T @ dR).reshape(3, 3)
    return dK, dQ, dV, dw0, deta


def test_matches_an_independent_matrix_derivation():
    rng = np.random.default_rng(41)
    gh, gw = 6, 9
    K, Q, V, w0, eta, dZ = _rand(rng, 2, 2, gh, gw, 5)
    got = oracle.dwconv3x3_fullbatch_bwd(K, Q, V, w0, eta, dZ, gh, gw)
    ref = _matrix_form(K, Q, V, w0, eta, dZ, gh, gw)
    for a, b in zip(got, ref):
        assert _rel(a, b) < 1e-12


def test_dq_is_torch_conv_transpose_with_the_updated_kernel():
    rng = np.random.default_rng(42)
    gh, gw, d = 7, 5, 6
    K, Q, V, w0, eta, dZ = _rand(rng, 1, 1, gh, gw, d)
    _, g = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    w1 = w0[0] - eta[0] * g[0, 0]
    _, dQ, _, _, _ = oracle.dwconv3x3_fullbatch_bwd(K, Q, V, w0, eta, dZ, gh, gw)
    img = torch.from_numpy(dZ[0, 0].reshape(gh, gw, d).transpose(2, 0, 1).copy())[None]
    ref = F.conv_transpose2d(img, torch.from_numpy(w1.copy())[:, None], padding=1, groups=d)
    ref = ref[0].numpy().transpose(1, 2, 0).reshape(gh * gw, d)
    assert _rel(dQ[0, 0], ref) < 1e-13


def test_zero_step_size_closed_form():
    rng = np.random.default_rng(43)
    gh, gw, d = 5, 8, 4
    K, Q, V, w0, eta, dZ = _rand(rng, 2, 1, gh, gw, d)
    eta[:] = 0.0
    dK, dQ, dV, dw0, deta = oracle.dwconv3x3_fullbatch_bwd(K, Q, V, w0, eta, dZ, gh, gw)
    assert np.max(np.abs(dK)) == 0.0 and np.max(np.abs(dV)) == 0.0
    # dw0 = dw1 = sum_p dZ[p] Q-window[p], deta = -<dw1, g>
    _, g = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    dw1 = np.zeros((d, 9))
    for b in range(2):
        for c in range(d):
            dw1[c] += _im2col(Q[b, 0, :, c], gh, gw).T @ dZ[b, 0, :, c]
    assert _rel(dw0[0].reshape(d, 9), dw1) < 1e-13
    de = 0.0
    for b in range(2):
        dw1b = np.stack([_im2col(Q[b, 0, :, c], gh, gw).T @ dZ[b, 0, :, c] for c in range(d)])
        de -= np.sum(dw1b * g[b, 0].reshape(d, 9))
    assert abs(deta[0] - de) < 1e-12 * max(1.0, abs(de))


def test_batch_sums_and_nonzero_dv():
    rng = np.random.default_rng(44)
    gh, gw, d = 4, 6, 3
    K, Q, V, w0, eta, dZ = _rand(rng, 3, 2, gh, gw, d)
    dK, dQ, dV, dw0, deta = oracle.dwconv3x3_fullbatch_bwd(K, Q, V, w0, eta, dZ, gh, gw)
    assert np.max(np.abs(dV)) > 1e-3  # the value view gets a gradient only through the update
    sw0, seta = np.zeros_like(dw0), np.zeros_like(deta)
    for b in range(3):
        r = oracle.dwconv3x3_fullbatch_bwd(K[b:b + 1], Q[b:b + 1], V[b:b + 1], w0, eta, dZ[b:b + 1], gh, gw)
        assert _rel(r[0], dK[b:b + 1]) == 0.0 and _rel(r[2], dV[b:b + 1]) == 0.0
        sw0 += r[3]
        seta += r[4]
    assert _rel(dw0, sw0) < 1e-14 and _rel(deta, seta) < 1e-14
