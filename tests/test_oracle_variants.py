"""Pins of the oracle's inner-training variants (no GPU).

  * Dot-product loss (ViT3 recipe): one step is linear attention plus the
    W0 term, Z = Q W0^T + (eta/N) Q K^T V, checked by numpy matmuls; its
    depthwise form is an im2col product; its gradients pass central finite
    differences of <dZ, Z> through the (pinned) forward.
  * Several full-batch steps (epochs): under L2 the iteration is affine,
    W_E = W* + (W0 - W*)(I - (2 eta/N) A)^E with W* = C A^{-1} (matrix
    power in numpy); under the dot loss W_E = W0 + E (eta/N) C; one step
    equals the single-step oracle.
  * One initial state per direction: equal copies give the shared-state
    scans; each single direction uses its own copy; the average is the
    mean of the two single-direction scans.
  * Gradient magnitude map: the Frobenius norm of the rank-one G_t equals
    2 ||W0 k - v|| ||k|| (dot: ||v|| ||k||); reconstructible values give 0.
"""
import numpy as np

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


def test_one_l2_step_equals_the_single_step_oracle():
    rng = np.random.default_rng(60)
    K, Q, V, W0, eta = _rand(rng, 2, 3, 50, 8)
    Z1, W = oracle.linear_fullbatch_ex(K, Q, V, W0, eta, oracle.L2, 1)
    Z0, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    assert _rel(Z1, Z0) < 1e-14
    assert _rel(W, W0[None] - eta[None, :, None, None] * G) < 1e-14


def test_dot_loss_one_step_is_linear_attention_plus_w0():
    rng = np.random.default_rng(61)
    B, H, N, d = 2, 2, 40, 8
    K, Q, V, W0, eta = _rand(rng, B, H, N, d)
    Z, W = oracle.linear_fullbatch_ex(K, Q, V, W0, eta, oracle.DOT, 1)
    for b in range(B):
        for h in range(H):
            ref = Q[b, h] @ W0[h].T + (eta[h] / N) * (Q[b, h] @ K[b, h].T) @ V[b, h]
            assert _rel(Z[b, h], ref) < 1e-13
            assert _rel(W[b, h], W0[h] + (eta[h] / N) * V[b, h].T @ K[b, h]) < 1e-13


def test_l2_epochs_follow_the_affine_closed_form():
    rng = np.random.default_rng(62)
    B, H, N, d = 1, 2, 60, 6
    K, Q, V, W0, _ = _rand(rng, B, H, N, d)
    eta = np.array([0.3, 0.8])
    for E in (2, 3, 7):
        Z, W = oracle.linear_fullbatch_ex(K, Q, V, W0, eta, oracle.L2, E)
        for h in range(H):
            A = K[0, h].T @ K[0, h]
            C = V[0, h].T @ K[0, h]
            Wstar = C @ np.linalg.inv(A)
            T = np.eye(d) - (2 * eta[h] / N) * A
            ref = Wstar + (W0[h] - Wstar) @ np.linalg.matrix_power(T, E)
            assert _rel(W[0, h], ref) < 1e-11
            assert _rel(Z[0, h], Q[0, h] @ ref.T) < 1e-11


def test_dot_epochs_repeat_the_constant_gradient():
    rng = np.random.default_rng(63)
    K, Q, V, W0, eta = _rand(rng, 2, 1, 30, 5)
    for E in (1, 4):
        _, W = oracle.linear_fullbatch_ex(K, Q, V, W0, eta, oracle.DOT, E)
        for b in range(2):
            ref = W0[0] + E * (eta[0] / 30) * V[b, 0].T @ K[b, 0]
            assert _rel(W[b, 0], ref) < 1e-13


def _fd_check(loss_fn, args, grads, h=1e-6, tol=1e-7):
    for a, gr in zip(args, grads):
        fd = np.empty_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            old = a[ix]
            a[ix] = old + h
            lp = loss_fn()
            a[ix] = old - h
            lm = loss_fn()
            a[ix] = old
            fd[ix] = (lp - lm) / (2 * h)
        assert _rel(gr, fd) < tol, (_rel(gr, fd), a.shape)


def test_dot_loss_linear_backward_finite_differences():
    rng = np.random.default_rng(64)
    K, Q, V, W0, eta = _rand(rng, 2, 2, 6, 4)
    dZ = rng.standard_normal(K.shape)
    grads = oracle.linear_fullbatch_bwd_ex(K, Q, V, W0, eta, dZ, oracle.DOT)
    args = [K, Q, V, W0, eta]
    _fd_check(lambda: float(np.sum(dZ * oracle.linear_fullbatch_ex(*args, oracle.DOT, 1)[0])), args, grads)
    # L2 through the same entry point is the pinned L2 backward
    g2 = oracle.linear_fullbatch_bwd_ex(K, Q, V, W0, eta, dZ, oracle.L2)
    g0 = oracle.linear_fullbatch_bwd(K, Q, V, W0, eta, dZ)
    for x, y in zip(g2, g0):
        assert _rel(x, y) == 0.0


def _im2col(X, gh, gw):
    img = np.zeros((gh + 2, gw + 2))
    img[1:-1, 1:-1] = X.reshape(gh, gw)
    cols = np.empty((gh * gw, 9))
    for i in range(3):
        for j in range(3):
            cols[:, 3 * i + j] = img[i:i + gh, j:j + gw].reshape(-1)
    return cols


def test_dot_loss_conv_step_is_an_im2col_product():
    rng = np.random.default_rng(65)
    B, H, gh, gw, d = 2, 1, 5, 7, 4
    K, Q, V, _, eta = _rand(rng, B, H, gh * gw, d)
    w0 = rng.standard_normal((H, d, 3, 3)) / 3.0
    Z, g = oracle.dwconv3x3_fullbatch_ex(K, Q, V, w0, eta, gh, gw, oracle.DOT)
    N = gh * gw
    for b in range(B):
        for c in range(d):
            XK = _im2col(K[b, 0, :, c], gh, gw)
            gr = -(1.0 / N) * XK.T @ V[b, 0, :, c]
            assert _rel(g[b, 0, c].reshape(9), gr) < 1e-13
            w1 = w0[0, c].reshape(9) - eta[0] * gr
            assert _rel(Z[b, 0, :, c], _im2col(Q[b, 0, :, c], gh, gw) @ w1) < 1e-13
    # L2 through the same entry point is the pinned L2 step
    Zl, gl = oracle.dwconv3x3_fullbatch_ex(K, Q, V, w0, eta, gh, gw, oracle.L2)
    Z0, g0 = oracle.dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    assert _rel(Zl, Z0) == 0.0 and _rel(gl, g0) == 0.0


def test_dot_loss_conv_backward_finite_differences():
    rng = np.random.default_rng(66)
    B, H, gh, gw, d = 1, 2, 4, 3, 3
    K, Q, V, _, eta = _rand(rng, B, H, gh * gw, d)
    w0 = rng.standard_normal((H, d, 3, 3)) / 3.0
    dZ = rng.standard_normal(K.shape)
    grads = oracle.dwconv3x3_fullbatch_bwd_ex(K, Q, V, w0, eta, dZ, gh, gw, oracle.DOT)
    args = [K, Q, V, w0, eta]
    _fd_check(lambda: float(np.sum(dZ * oracle.dwconv3x3_fullbatch_ex(*args, gh, gw, oracle.DOT)[0])), args,
              grads)


def test_one_initial_state_per_direction():
    rng = np.random.default_rng(67)
    B, H, N, d, b = 2, 2, 37, 6, 5
    K, Q, V, W0, eta = _rand(rng, B, H, N, d)
    W1 = rng.standard_normal((H, d, d)) / np.sqrt(d)
    same = np.stack([W0, W0])
    for mode in (0, 1, 2):
        assert _rel(oracle.linear_minibatch_2w0(K, Q, V, same, eta, b, mode),
                    oracle.linear_minibatch(K, Q, V, W0, eta, b, mode)) == 0.0
    two = np.stack([W0, W1])
    f = oracle.linear_minibatch_2w0(K, Q, V, two, eta, b, 1)
    r = oracle.linear_minibatch_2w0(K, Q, V, two, eta, b, 2)
    assert _rel(f, oracle.linear_minibatch(K, Q, V, W0, eta, b, 1)) == 0.0
    assert _rel(r, oracle.linear_minibatch(K, Q, V, W1, eta, b, 2)) == 0.0
    assert _rel(oracle.linear_minibatch_2w0(K, Q, V, two, eta, b, 0), 0.5 * (f + r)) < 1e-15


def test_gradient_magnitude_map_closed_form():
    rng = np.random.default_rng(68)
    K, _, V, W0, _ = _rand(rng, 2, 3, 25, 7)
    m = oracle.linear_gradient_magnitude(K, V, W0, oracle.L2)
    r = np.einsum("hoc,bhnc->bhno", W0, K) - V
    ref = 2 * np.linalg.norm(r, axis=-1) * np.linalg.norm(K, axis=-1)
    assert _rel(m, ref) < 1e-13
    md = oracle.linear_gradient_magnitude(K, V, W0, oracle.DOT)
    assert _rel(md, np.linalg.norm(V, axis=-1) * np.linalg.norm(K, axis=-1)) < 1e-13
    Vr = np.einsum("hoc,bhnc->bhno", W0, K)
    assert np.max(oracle.linear_gradient_magnitude(K, Vr, W0, oracle.L2)) < 1e-13
