"""Pins of the oracle's mini-batch scan backward and of its two-layer SiLU
MLP inner model (no GPU).

Scan backward: central finite differences of L = <dZ, Z> through the
(separately pinned) scan forward, for every entry of K, Q, V, W0 and eta, in
all three modes with a ragged last mini-batch, and at b = 1 and b = N; with
b = N and dZ only on the last token the gradient is the full-batch step's
(whose backward is pinned by its own finite differences); the averaged mode
is the mean of the two single-direction gradients.

MLP: the full-batch gradients equal torch autograd's (a library routine, in
fp64) and central finite differences of the mean loss; the output is the
updated model applied to q, computed here with numpy.
"""
import numpy as np
import torch

import oracle


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _rand(rng, B, H, N, d):
    K = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    Q = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    V = rng.standard_normal((B, H, N, d))
    W0 = rng.standard_normal((H, d, d)) / np.sqrt(d)
    eta = rng.uniform(0.5, 2.0, size=H)
    return K, Q, V, W0, eta


def _fd(loss, args, grads, h=1e-6, tol=1e-7):
    for a, gr in zip(args, grads):
        fd = np.empty_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = a[ix]
            a[ix] = old + h
            lp = loss()
            a[ix] = old - h
            lm = loss()
            a[ix] = old
            fd[ix] = (lp - lm) / (2 * h)
        assert _rel(gr, fd) < tol, (_rel(gr, fd), a.shape)


def test_scan_backward_finite_differences_all_modes():
    rng = np.random.default_rng(80)
    for mode in (0, 1, 2):
        for N, b in ((7, 3), (5, 1), (6, 6)):
            K, Q, V, W0, eta = _rand(rng, 1, 2, N, 4)
            dZ = rng.standard_normal(K.shape)
            grads = oracle.linear_minibatch_bwd(K, Q, V, W0, eta, dZ, b, mode)
            args = [K, Q, V, W0, eta]
            _fd(lambda: float(np.sum(dZ * oracle.linear_minibatch(*args, b, mode))), args, grads)


def test_scan_backward_with_one_minibatch_is_the_full_batch_step_at_the_last_token():
    rng = np.random.default_rng(81)
    B, H, N, d = 2, 2, 20, 6
    K, Q, V, W0, eta = _rand(rng, B, H, N, d)
    dZ = np.zeros(K.shape)
    dZ[:, :, -1] = rng.standard_normal((B, H, d))
    got = oracle.linear_minibatch_bwd(K, Q, V, W0, eta, dZ, N, 1)
    ref = oracle.linear_fullbatch_bwd(K, Q, V, W0, eta, dZ)
    for x, y in zip(got, ref):
        assert _rel(x, y) < 1e-12


def test_scan_backward_average_is_the_mean_of_the_directions():
    rng = np.random.default_rng(82)
    K, Q, V, W0, eta = _rand(rng, 2, 1, 23, 5)
    dZ = rng.standard_normal(K.shape)
    a = oracle.linear_minibatch_bwd(K, Q, V, W0, eta, dZ, 4, 0)
    f = oracle.linear_minibatch_bwd(K, Q, V, W0, eta, dZ, 4, 1)
    r = oracle.linear_minibatch_bwd(K, Q, V, W0, eta, dZ, 4, 2)
    for x, y, z in zip(a, f, r):
        assert _rel(x, 0.5 * (y + z)) < 1e-13
    assert np.max(np.abs(a[2])) > 1e-3  # the value view's gradient flows through the updates


def _mlp_rand(rng, B, H, N, d, r):
    K, Q, V, _, eta = _rand(rng, B, H, N, d)
    W1 = rng.standard_normal((H, r * d, d)) / np.sqrt(d)
    W2 = rng.standard_normal((H, d, r * d)) / np.sqrt(r * d)
    return K, Q, V, W1, W2, eta


def test_mlp_gradients_equal_torch_autograd():
    rng = np.random.default_rng(83)
    for r in (1, 2, 4):
        K, Q, V, W1, W2, eta = _mlp_rand(rng, 2, 2, 30, 8, r)
        _, G1, G2 = oracle.mlp_fullbatch(K, Q, V, W1, W2, eta)
        for b in range(2):
            for h in range(2):
                w1 = torch.tensor(W1[h], requires_grad=True)
                w2 = torch.tensor(W2[h], requires_grad=True)
                k, v = torch.tensor(K[b, h]), torch.tensor(V[b, h])
                out = torch.nn.functional.silu(k @ w1.T) @ w2.T
                loss = ((out - v) ** 2).sum(dim=1).mean()
                loss.backward()
                assert _rel(G1[b, h], w1.grad.numpy()) < 1e-12
                assert _rel(G2[b, h], w2.grad.numpy()) < 1e-12


def test_mlp_gradients_finite_differences_and_output():
    rng = np.random.default_rng(84)
    K, Q, V, W1, W2, eta = _mlp_rand(rng, 1, 1, 9, 4, 2)
    Z, G1, G2 = oracle.mlp_fullbatch(K, Q, V, W1, W2, eta)
    k, v = K[0, 0], V[0, 0]

    def loss():
        a = k @ W1[0].T
        a = a / (1 + np.exp(-a))
        return float(np.mean(np.sum((a @ W2[0].T - v) ** 2, axis=1)))

    _fd(loss, [W1, W2], [G1[0], G2[0]])
    w1n, w2n = W1[0] - eta[0] * G1[0, 0], W2[0] - eta[0] * G2[0, 0]
    a = Q[0, 0] @ w1n.T
    assert _rel(Z[0, 0], (a / (1 + np.exp(-a))) @ w2n.T) < 1e-13
