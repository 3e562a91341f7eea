"""Pins of the oracle's backward through the full-batch linear step (no GPU).

The oracle differentiates the residual (per-token) form in reverse mode; the
pins are central finite differences of L = sum(dZ * Z) through the (already
pinned) forward oracle, an independent Gram-form expression of the same
gradients, and the mixed-derivative property the ViT3 article stresses
(values receive a gradient through the inner update).
"""
import numpy as np

import oracle


def _rand(rng, B, H, N, d):
    K = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    Q = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    V = rng.standard_normal((B, H, N, d))
    W0 = rng.standard_normal((H, d, d)) / np.sqrt(d)
    eta = rng.uniform(0.5, 2.0, size=H)
    dZ = rng.standard_normal((B, H, N, d))
    return K, Q, V, W0, eta, dZ


def _L(K, Q, V, W0, eta, dZ):
    Z, _ = oracle.linear_fullbatch(K, Q, V, W0, eta)
    return float(np.sum(Z * dZ))


def _fd_check(args, grads, names, idx_per, rng, h=1e-5, tol=1e-6):
    args = [a.copy() for a in args]
    for name, gi in zip(names, range(len(grads))):
        pos = {"K": 0, "Q": 1, "V": 2, "W0": 3, "eta": 4}[name]
        x = args[pos]
        flat = x.reshape(-1)
        picks = rng.choice(flat.size, size=min(idx_per, flat.size), replace=False)
        g = grads[gi].reshape(-1)
        scale = max(np.max(np.abs(g)), 1e-30)
        for p in picks:
            old = flat[p]
            flat[p] = old + h
            lp = _L(*args)
            flat[p] = old - h
            lm = _L(*args)
            flat[p] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[p]) <= tol * scale, (name, p, fd, g[p])


def test_finite_differences_full_slice_shape():
    # B=1, H=1, N=64, d=64: the slice the fp32 GPU check also uses.
    rng = np.random.default_rng(40)
    K, Q, V, W0, eta, dZ = _rand(rng, 1, 1, 64, 64)
    dK, dQ, dV, dW0, deta = oracle.linear_fullbatch_bwd(K, Q, V, W0, eta, dZ)
    _fd_check((K, Q, V, W0, eta, dZ), (dK, dQ, dV, dW0, deta),
              ("K", "Q", "V", "W0", "eta"), 40, rng)


def test_finite_differences_every_entry_small():
    rng = np.random.default_rng(41)
    K, Q, V, W0, eta, dZ = _rand(rng, 2, 2, 7, 4)
    dK, dQ, dV, dW0, deta = oracle.linear_fullbatch_bwd(K, Q, V, W0, eta, dZ)
    _fd_check((K, Q, V, W0, eta, dZ), (dK, dQ, dV, dW0, deta),
              ("K", "Q", "V", "W0", "eta"), 10 ** 6, rng)


def test_matches_gram_form():
    # dW1 = dZ^T Q, beta = 2 eta / N, M = W0^T dW1 + dW1^T W0:
    # dQ = dZ W1 ; dK = beta (V dW1 - K M) ; dV = beta K dW1^T ;
    # dW0 = sum_b dW1 (I - beta A) ; deta = -sum_b <dW1, G>.
    rng = np.random.default_rng(42)
    B, H, N, d = 3, 2, 45, 16
    K, Q, V, W0, eta, dZ = _rand(rng, B, H, N, d)
    dK, dQ, dV, dW0, deta = oracle.linear_fullbatch_bwd(K, Q, V, W0, eta, dZ)
    rdW0 = np.zeros((H, d, d))
    rdeta = np.zeros(H)
    for b in range(B):
        for h in range(H):
            k, q, v, dz = K[b, h], Q[b, h], V[b, h], dZ[b, h]
            A = k.T @ k
            C = v.T @ k
            beta = 2.0 * eta[h] / N
            G = (2.0 / N) * (W0[h] @ A - C)
            W1 = W0[h] - eta[h] * G
            dW1 = dz.T @ q
            M = W0[h].T @ dW1 + dW1.T @ W0[h]
            np.testing.assert_allclose(dQ[b, h], dz @ W1, rtol=0, atol=1e-12)
            np.testing.assert_allclose(dK[b, h], beta * (v @ dW1 - k @ M), rtol=0, atol=1e-12)
            np.testing.assert_allclose(dV[b, h], beta * k @ dW1.T, rtol=0, atol=1e-12)
            rdW0[h] += dW1 @ (np.eye(d) - beta * A)
            rdeta[h] -= np.sum(dW1 * G)
    np.testing.assert_allclose(dW0, rdW0, rtol=0, atol=1e-11)
    np.testing.assert_allclose(deta, rdeta, rtol=1e-12, atol=0)


def test_values_receive_gradient_through_the_update():
    # The mixed second derivative of the L2 loss is non-zero, so dV != 0;
    # with eta = 0 the update is switched off and dV vanishes exactly.
    rng = np.random.default_rng(43)
    K, Q, V, W0, eta, dZ = _rand(rng, 1, 1, 12, 8)
    _, _, dV, _, _ = oracle.linear_fullbatch_bwd(K, Q, V, W0, eta, dZ)
    assert np.max(np.abs(dV)) > 1e-3
    _, _, dV0, _, _ = oracle.linear_fullbatch_bwd(K, Q, V, W0, np.zeros(1), dZ)
    assert np.max(np.abs(dV0)) == 0.0
