"""Pins of the oracle's mini-batch bidirectional scans (no GPU).

Closed forms and special cases: b = N is one full-batch step; b = 1 is plain
per-token gradient descent; the reverse scan is the forward scan of the
flipped sequence; the chunk counts of the pages' worked example; and an
independent chunk-matrix ("dual") form of the same recurrence at b = 16 with
a ragged last mini-batch.
"""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chunk_counts.txt")


def _rand(rng, B, H, N, d, unit=False):
    if unit:
        K = rng.standard_normal((B, H, N, d)); K /= np.linalg.norm(K, axis=-1, keepdims=True)
        Q = rng.standard_normal((B, H, N, d)); Q /= np.linalg.norm(Q, axis=-1, keepdims=True)
    else:
        K = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
        Q = rng.standard_normal((B, H, N, d)) / np.sqrt(d)
    V = rng.standard_normal((B, H, N, d))
    W0 = rng.standard_normal((H, d, d)) / np.sqrt(d)
    eta = rng.uniform(0.5, 2.0, size=H)
    return K, Q, V, W0, eta


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_chunk_counts_match_worked_example():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert rows
    for N, b, steps, last in (map(int, r) for r in rows):
        assert oracle.num_chunks(N, b) == steps
        assert N - (steps - 1) * b == last
    # both directions together: 26 state writes at N=196, b=16
    assert 2 * oracle.num_chunks(196, 16) == 26


def test_full_batch_size_equals_full_batch_step():
    rng = np.random.default_rng(30)
    K, Q, V, W0, eta = _rand(rng, 1, 2, 40, 8)
    Zf = oracle.linear_minibatch(K, Q, V, W0, eta, 40, oracle.FORWARD_ONLY)
    Zfb, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    # after the last token the forward state is W0 - eta G
    assert _rel(Zf[:, :, -1], Zfb[:, :, -1]) < 1e-13
    # reverse scan: its last token is position 0
    Zr = oracle.linear_minibatch(K, Q, V, W0, eta, 40, oracle.BACKWARD_ONLY)
    assert _rel(Zr[:, :, 0], Zfb[:, :, 0]) < 1e-13


def test_full_batch_size_bidirectional_closed_form():
    # One mini-batch per direction: averaging the two states at token t gives
    # (W0 + W1)/2 - (eta/N) r_t k_t^T with r_t = W0 k_t - v_t.
    rng = np.random.default_rng(31)
    K, Q, V, W0, eta = _rand(rng, 1, 1, 25, 6)
    Z = oracle.linear_minibatch(K, Q, V, W0, eta, 25, oracle.FORWARD_BACKWARD_AVG)
    _, G = oracle.linear_fullbatch(K, Q, V, W0, eta)
    W1 = W0[0] - eta[0] * G[0, 0]
    for t in range(25):
        k, v, q = K[0, 0, t], V[0, 0, t], Q[0, 0, t]
        r = W0[0] @ k - v
        Wt = 0.5 * (W0[0] + W1) - (eta[0] / 25) * np.outer(r, k)
        assert _rel(Z[0, 0, t], Wt @ q) < 1e-12


def test_unit_batch_is_per_token_gradient_descent():
    rng = np.random.default_rng(32)
    K, Q, V, W0, eta = _rand(rng, 1, 1, 30, 5)
    Z = oracle.linear_minibatch(K, Q, V, W0, eta, 1, oracle.FORWARD_ONLY)
    W = W0[0].copy()
    for t in range(30):
        k, v, q = K[0, 0, t], V[0, 0, t], Q[0, 0, t]
        W = W - eta[0] * 2.0 * np.outer(W @ k - v, k)
        assert _rel(Z[0, 0, t], W @ q) < 1e-12


def test_reverse_scan_is_flipped_forward_scan():
    rng = np.random.default_rng(33)
    K, Q, V, W0, eta = _rand(rng, 2, 2, 37, 8)
    Zr = oracle.linear_minibatch(K, Q, V, W0, eta, 16, oracle.BACKWARD_ONLY)
    fl = lambda x: x[:, :, ::-1].copy()
    Zf = oracle.linear_minibatch(fl(K), fl(Q), fl(V), W0, eta, 16, oracle.FORWARD_ONLY)
    assert _rel(Zr, fl(Zf)) < 1e-14


def test_bidirectional_is_average_of_directions():
    rng = np.random.default_rng(34)
    K, Q, V, W0, eta = _rand(rng, 1, 3, 21, 8)
    Za = oracle.linear_minibatch(K, Q, V, W0, eta, 4, oracle.FORWARD_BACKWARD_AVG)
    Zf = oracle.linear_minibatch(K, Q, V, W0, eta, 4, oracle.FORWARD_ONLY)
    Zr = oracle.linear_minibatch(K, Q, V, W0, eta, 4, oracle.BACKWARD_ONLY)
    assert _rel(Za, 0.5 * (Zf + Zr)) < 1e-15


def _dual_form_forward(K, Q, V, W0, eta, b):
    """Chunk-matrix form of one forward scan of one slice:
    R = K_c W^T - V_c ; Z_c = Q_c W^T - a tril(Q_c K_c^T) R ; W -= a R^T K_c
    with a = 2 eta / n_c (derived from the per-token definition)."""
    N = K.shape[0]
    W = W0.copy()
    Z = np.zeros_like(Q)
    for c0 in range(0, N, b):
        Kc, Vc, Qc = K[c0:c0 + b], V[c0:c0 + b], Q[c0:c0 + b]
        a = 2.0 * eta / Kc.shape[0]
        R = Kc @ W.T - Vc
        Z[c0:c0 + b] = Qc @ W.T - a * np.tril(Qc @ Kc.T) @ R
        W = W - a * R.T @ Kc
    return Z


def test_matches_chunk_matrix_form_with_ragged_tail():
    rng = np.random.default_rng(35)
    K, Q, V, W0, eta = _rand(rng, 1, 2, 50, 16, unit=True)
    Z = oracle.linear_minibatch(K, Q, V, W0, eta, 16, oracle.FORWARD_ONLY)
    for h in range(2):
        ref = _dual_form_forward(K[0, h], Q[0, h], V[0, h], W0[h], eta[h], 16)
        assert _rel(Z[0, h], ref) < 1e-12


def test_long_scan_stays_bounded_with_unit_keys():
    # 400 mini-batches at the 1280x1280 shape per slice, eta = 1, unit keys:
    # the normalised update contracts, so outputs stay O(1).
    rng = np.random.default_rng(36)
    K, Q, V, W0, _ = _rand(rng, 1, 1, 6400, 64, unit=True)
    Z = oracle.linear_minibatch(K, Q, V, W0, np.ones(1), 16, oracle.FORWARD_BACKWARD_AVG)
    assert np.all(np.isfinite(Z)) and np.max(np.abs(Z)) < 10.0
