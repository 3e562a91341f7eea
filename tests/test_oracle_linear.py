"""Pins of the oracle's full-batch linear step (no GPU).

Each test fixes the oracle to something other than itself: a closed form of
the method (zero update when V = W0 K, linear attention when W0 = 0,
identity when eta = 0), the Gram rewriting of the gradient, central finite
differences of the loss, and invariances.  A dropped term, a wrong sign, a
wrong scale (1/N vs 2/N) or a transposed operand fails at least one of them.
"""
import numpy as np
import pytest

import oracle


def _rand(rng, B, H, N, d):
    K = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    Q = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    V = rng.standard_normal((B, H, N, d))
    W0 = rng.standard_normal((H, d, d)) / np.sqrt(d)
    eta = rng.uniform(0.5, 2.0, size=H)
    return K, Q, V, W0, eta


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_reconstructible_values_give_zero_update():
    # V = W0 K exactly: every residual vanishes, so G = 0 and z = W0 q.
    rng = np.random.default_rng(10)
    K, Q, _, W0, eta = _rand(rng, 2, 3, 37, 16)
    V = np.einsum("hrc,bhnc->bhnr", W0, K)
    Z, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    assert np.max(np.abs(G)) < 1e-14
    ref = np.einsum("hrc,bhnc->bhnr", W0, Q)
    assert _rel(Z, ref) < 1e-13


def test_zero_init_is_linear_attention():
    # W0 = 0: W1 = (2 eta / N) V^T K, so Z = (2 eta / N) (Q K^T) V, which is
    # (unnormalised) linear attention -- the "one step equals gated linear
    # attention" remark of the Vision-TTT notes.
    rng = np.random.default_rng(11)
    K, Q, V, W0, eta = _rand(rng, 2, 2, 50, 16)
    W0[:] = 0.0
    Z, _ = oracle.linear_fullbatch(K, Q, V, W0, eta)
    N = K.shape[2]
    for b in range(2):
        for h in range(2):
            att = (Q[b, h] @ K[b, h].T) @ V[b, h]
            assert _rel(Z[b, h], (2.0 * eta[h] / N) * att) < 1e-13


def test_zero_step_is_identity_update():
    rng = np.random.default_rng(12)
    K, Q, V, W0, eta = _rand(rng, 1, 2, 20, 8)
    eta[:] = 0.0
    Z, _ = oracle.linear_fullbatch(K, Q, V, W0, eta)
    assert _rel(Z, np.einsum("hrc,bhnc->bhnr", W0, Q)) < 1e-14


def test_gradient_equals_gram_form():
    # (2/N) sum (W0 k - v) k^T == (2/N) (W0 K^T K - V^T K)
    rng = np.random.default_rng(13)
    K, Q, V, W0, eta = _rand(rng, 2, 2, 61, 64)
    _, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    N = K.shape[2]
    for b in range(2):
        for h in range(2):
            A = K[b, h].T @ K[b, h]
            C = V[b, h].T @ K[b, h]
            assert _rel(G[b, h], (2.0 / N) * (W0[h] @ A - C)) < 1e-12


def _loss(W, K, V):
    R = K @ W.T - V
    return np.mean(np.sum(R * R, axis=1))


def test_gradient_matches_finite_differences():
    # G is the gradient of the token-mean L2 loss at W0 (every entry, d = 6).
    rng = np.random.default_rng(14)
    K, Q, V, W0, eta = _rand(rng, 1, 1, 23, 6)
    _, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    h = 1e-6
    fd = np.zeros_like(W0[0])
    for r in range(6):
        for c in range(6):
            Wp = W0[0].copy(); Wp[r, c] += h
            Wm = W0[0].copy(); Wm[r, c] -= h
            fd[r, c] = (_loss(Wp, K[0, 0], V[0, 0]) - _loss(Wm, K[0, 0], V[0, 0])) / (2 * h)
    assert _rel(G[0, 0], fd) < 1e-7


def test_output_uses_updated_weights():
    # z_i = W1 q_i with W1 = W0 - eta G, checked row by row.
    rng = np.random.default_rng(15)
    K, Q, V, W0, eta = _rand(rng, 1, 2, 9, 5)
    Z, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    for h in range(2):
        W1 = W0[h] - eta[h] * G[0, h]
        for i in range(9):
            assert _rel(Z[0, h, i], W1 @ Q[0, h, i]) < 1e-13


def test_small_step_decreases_loss():
    rng = np.random.default_rng(16)
    K, Q, V, W0, eta = _rand(rng, 1, 1, 40, 8)
    _, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    W1 = W0[0] - 0.05 * G[0, 0]
    assert _loss(W1, K[0, 0], V[0, 0]) < _loss(W0[0], K[0, 0], V[0, 0])


def test_token_permutation_leaves_update_unchanged():
    rng = np.random.default_rng(17)
    K, Q, V, W0, eta = _rand(rng, 1, 1, 33, 16)
    _, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    p = rng.permutation(33)
    _, Gp = oracle.linear_fullbatch(K[:, :, p], Q, V[:, :, p], W0, eta)
    assert _rel(Gp, G) < 1e-13


def test_heads_and_images_are_independent():
    rng = np.random.default_rng(18)
    K, Q, V, W0, eta = _rand(rng, 3, 2, 17, 8)
    Z, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    Z1, G1 = oracle.linear_fullbatch(K[1:2, 1:2], Q[1:2, 1:2], V[1:2, 1:2], W0[1:2], eta[1:2])
    assert np.array_equal(Z[1, 1], Z1[0, 0]) and np.array_equal(G[1, 1], G1[0, 0])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(19)
    K, Q, V, W0, eta = _rand(rng, 2, 3, 29, 16)
    Za, Ga = oracle.linear_fullbatch(K, Q, V, W0, eta, threads=1)
    Zb, Gb = oracle.linear_fullbatch(K, Q, V, W0, eta, threads=4)
    assert np.array_equal(Za, Zb) and np.array_equal(Ga, Gb)


def test_rejects_bad_shape():
    with pytest.raises(ValueError):
        oracle.linear_fullbatch(np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 0, 4)),
                                np.zeros((1, 1, 0, 4)), np.zeros((1, 4, 4)), np.ones(1))
