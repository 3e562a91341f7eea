"""fp64 CPU oracle of the multi-head TTT layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only users.  The product package never
imports this module, and this module never imports the product package: the
two share no code.  Callers hand in the exact (already quantised) inputs as
arrays; they are widened to float64 here and every result is float64.

The arithmetic lives in ``ttt_oracle.c`` (plain loops, OpenMP over
independent slices), whose header lists the passages of the pages each
function follows and the readings taken where the pages are silent.

Every function below is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, finite differences,
brute-force im2col gradients and the pages' worked example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ttt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libttt_oracle.so")
_lib = None

FORWARD_BACKWARD_AVG = 0
FORWARD_ONLY = 1
BACKWARD_ONLY = 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_linear_fullbatch.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_dwconv3x3_fullbatch.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_linear_minibatch.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_linear_fullbatch_bwd.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp,
                                                    dp, dp, dp, dp, dp, i]
        lib.oracle_dwconv3x3_fullbatch_bwd.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp,
                                                       dp, dp, dp, dp, dp, i]
        lib.oracle_linear_fullbatch_ex.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_linear_fullbatch_bwd_ex.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp,
                                                       dp, dp, dp, dp, dp, i]
        lib.oracle_dwconv3x3_fullbatch_ex.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_dwconv3x3_fullbatch_bwd_ex.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp,
                                                          dp, dp, dp, dp, dp, i]
        lib.oracle_linear_minibatch_2w0.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_linear_gradient_magnitude.argtypes = [i, i, i, i, i, dp, dp, dp, dp, i]
        for f in (lib.oracle_linear_fullbatch_ex, lib.oracle_linear_fullbatch_bwd_ex,
                  lib.oracle_dwconv3x3_fullbatch_ex, lib.oracle_dwconv3x3_fullbatch_bwd_ex,
                  lib.oracle_linear_minibatch_2w0, lib.oracle_linear_gradient_magnitude):
            f.restype = ctypes.c_int
        lib.oracle_linear_minibatch_bwd.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp,
                                                    dp, dp, dp, dp, dp, i]
        lib.oracle_mlp_fullbatch.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_linear_minibatch_bwd.restype = ctypes.c_int
        lib.oracle_mlp_fullbatch.restype = ctypes.c_int
        lib.oracle_num_chunks.argtypes = [i, i]
        lib.oracle_max_threads.argtypes = []
        for f in (lib.oracle_linear_fullbatch, lib.oracle_dwconv3x3_fullbatch,
                  lib.oracle_linear_minibatch, lib.oracle_linear_fullbatch_bwd,
                  lib.oracle_num_chunks, lib.oracle_max_threads, lib.oracle_dwconv3x3_fullbatch_bwd):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(rc, name):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % name)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def num_chunks(N: int, b: int) -> int:
    """Mini-batches per scan direction: ceil(N / b)."""
    rc = _load().oracle_num_chunks(int(N), int(b))
    if rc < 0:
        raise ValueError("bad N or b")
    return rc


def linear_fullbatch(K, Q, V, W0, eta, threads: int = 0):
    """One full-batch L2 step of the linear inner model, then z = W1 q.

    K, Q, V: [B,H,N,d]; W0: [H,d,d]; eta: [H].  Returns (Z, G) in float64,
    Z: [B,H,N,d], G: [B,H,d,d] (the full-batch gradient at W0).
    """
    K, Q, V, W0, eta = map(_f64, (K, Q, V, W0, eta))
    B, H, N, d = K.shape
    Z = np.empty_like(K)
    G = np.empty((B, H, d, d))
    _check(_load().oracle_linear_fullbatch(B, H, N, d, _p(K), _p(Q), _p(V), _p(W0), _p(eta),
                                           _p(Z), _p(G), int(threads)), "linear_fullbatch")
    return Z, G


def dwconv3x3_fullbatch(K, Q, V, w0, eta, grid_h: int, grid_w: int, threads: int = 0):
    """One full-batch L2 step of the depthwise 3x3 inner model, then apply.

    K, Q, V: [B,H,N,d] with N = grid_h*grid_w (row-major grid); w0: [H,d,3,3];
    eta: [H].  Returns (Z, g): Z [B,H,N,d], g [B,H,d,3,3].
    """
    K, Q, V, w0, eta = map(_f64, (K, Q, V, w0, eta))
    B, H, N, d = K.shape
    if grid_h * grid_w != N:
        raise ValueError("grid_h*grid_w != N")
    Z = np.empty_like(K)
    g = np.empty((B, H, d, 3, 3))
    _check(_load().oracle_dwconv3x3_fullbatch(B, H, grid_h, grid_w, d, _p(K), _p(Q), _p(V),
                                              _p(w0), _p(eta), _p(Z), _p(g), int(threads)),
           "dwconv3x3_fullbatch")
    return Z, g


def linear_minibatch(K, Q, V, W0, eta, minibatch: int, mode: int = FORWARD_BACKWARD_AVG,
                     threads: int = 0):
    """Causal mini-batch scans of the linear inner model.

    mode 0 averages the forward scan and the reverse scan (mapped back to
    token positions); 1 and 2 return one direction.  Returns Z [B,H,N,d].
    """
    K, Q, V, W0, eta = map(_f64, (K, Q, V, W0, eta))
    B, H, N, d = K.shape
    Z = np.empty_like(K)
    _check(_load().oracle_linear_minibatch(B, H, N, d, int(minibatch), int(mode), _p(K), _p(Q),
                                           _p(V), _p(W0), _p(eta), _p(Z), int(threads)),
           "linear_minibatch")
    return Z


def linear_fullbatch_bwd(K, Q, V, W0, eta, dZ, threads: int = 0):
    """Gradients of sum(dZ * Z) through the full-batch linear layer.

    Returns (dK, dQ, dV, dW0, deta); dW0 [H,d,d] and deta [H] are summed over
    the batch.
    """
    K, Q, V, W0, eta, dZ = map(_f64, (K, Q, V, W0, eta, dZ))
    B, H, N, d = K.shape
    dK = np.empty_like(K)
    dQ = np.empty_like(K)
    dV = np.empty_like(K)
    dW0 = np.empty((H, d, d))
    deta = np.empty((H,))
    _check(_load().oracle_linear_fullbatch_bwd(B, H, N, d, _p(K), _p(Q), _p(V), _p(W0), _p(eta),
                                               _p(dZ), _p(dK), _p(dQ), _p(dV), _p(dW0),
                                               _p(deta), int(threads)), "linear_fullbatch_bwd")
    return dK, dQ, dV, dW0, deta


def dwconv3x3_fullbatch_bwd(K, Q, V, w0, eta, dZ, grid_h: int, grid_w: int, threads: int = 0):
    """Gradients of sum(dZ * Z) through the depthwise 3x3 full-batch step.

    Returns (dK, dQ, dV, dw0, deta); dw0 [H,d,3,3] and deta [H] are summed
    over the batch.
    """
    K, Q, V, w0, eta, dZ = map(_f64, (K, Q, V, w0, eta, dZ))
    B, H, N, d = K.shape
    if grid_h * grid_w != N:
        raise ValueError("grid_h*grid_w != N")
    dK = np.empty_like(K)
    dQ = np.empty_like(K)
    dV = np.empty_like(K)
    dw0 = np.empty((H, d, 3, 3))
    deta = np.empty((H,))
    _check(_load().oracle_dwconv3x3_fullbatch_bwd(B, H, grid_h, grid_w, d, _p(K), _p(Q), _p(V), _p(w0),
                                                  _p(eta), _p(dZ), _p(dK), _p(dQ), _p(dV), _p(dw0),
                                                  _p(deta), int(threads)), "dwconv3x3_fullbatch_bwd")
    return dK, dQ, dV, dw0, deta


L2 = 0
DOT = 1


def linear_fullbatch_ex(K, Q, V, W0, eta, loss: int = L2, steps: int = 1, threads: int = 0):
    """`steps` full-batch gradient steps of the linear inner model under the
    L2 or dot-product loss, then z = W q.  Returns (Z, W) with W [B,H,d,d]
    the final inner weights."""
    K, Q, V, W0, eta = map(_f64, (K, Q, V, W0, eta))
    B, H, N, d = K.shape
    Z = np.empty_like(K)
    W = np.empty((B, H, d, d))
    _check(_load().oracle_linear_fullbatch_ex(B, H, N, d, int(loss), int(steps), _p(K), _p(Q), _p(V), _p(W0),
                                              _p(eta), _p(Z), _p(W), int(threads)), "linear_fullbatch_ex")
    return Z, W


def linear_fullbatch_bwd_ex(K, Q, V, W0, eta, dZ, loss: int = L2, threads: int = 0):
    """linear_fullbatch_bwd under the L2 or dot-product loss."""
    K, Q, V, W0, eta, dZ = map(_f64, (K, Q, V, W0, eta, dZ))
    B, H, N, d = K.shape
    out = [np.empty_like(K) for _ in range(3)] + [np.empty((H, d, d)), np.empty((H,))]
    _check(_load().oracle_linear_fullbatch_bwd_ex(B, H, N, d, int(loss), _p(K), _p(Q), _p(V), _p(W0), _p(eta),
                                                  _p(dZ), *(_p(o) for o in out), int(threads)),
           "linear_fullbatch_bwd_ex")
    return tuple(out)


def dwconv3x3_fullbatch_ex(K, Q, V, w0, eta, grid_h: int, grid_w: int, loss: int = L2, threads: int = 0):
    """dwconv3x3_fullbatch under the L2 or dot-product loss.  Returns (Z, g)."""
    K, Q, V, w0, eta = map(_f64, (K, Q, V, w0, eta))
    B, H, N, d = K.shape
    if grid_h * grid_w != N:
        raise ValueError("grid_h*grid_w != N")
    Z = np.empty_like(K)
    g = np.empty((B, H, d, 3, 3))
    _check(_load().oracle_dwconv3x3_fullbatch_ex(B, H, grid_h, grid_w, d, int(loss), _p(K), _p(Q), _p(V),
                                                 _p(w0), _p(eta), _p(Z), _p(g), int(threads)),
           "dwconv3x3_fullbatch_ex")
    return Z, g


def dwconv3x3_fullbatch_bwd_ex(K, Q, V, w0, eta, dZ, grid_h: int, grid_w: int, loss: int = L2,
                               threads: int = 0):
    """dwconv3x3_fullbatch_bwd under the L2 or dot-product loss."""
    K, Q, V, w0, eta, dZ = map(_f64, (K, Q, V, w0, eta, dZ))
    B, H, N, d = K.shape
    if grid_h * grid_w != N:
        raise ValueError("grid_h*grid_w != N")
    out = [np.empty_like(K) for _ in range(3)] + [np.empty((H, d, 3, 3)), np.empty((H,))]
    _check(_load().oracle_dwconv3x3_fullbatch_bwd_ex(B, H, grid_h, grid_w, d, int(loss), _p(K), _p(Q), _p(V),
                                                     _p(w0), _p(eta), _p(dZ), *(_p(o) for o in out),
                                                     int(threads)), "dwconv3x3_fullbatch_bwd_ex")
    return tuple(out)


def linear_minibatch_2w0(K, Q, V, W0, eta, minibatch: int, mode: int = FORWARD_BACKWARD_AVG,
                         threads: int = 0):
    """linear_minibatch with one initial state per direction: W0 [2,H,d,d]
    (forward scan from W0[0], reverse scan from W0[1])."""
    K, Q, V, W0, eta = map(_f64, (K, Q, V, W0, eta))
    B, H, N, d = K.shape
    if W0.shape != (2, H, d, d):
        raise ValueError("W0 must be [2,H,d,d]")
    Z = np.empty_like(K)
    _check(_load().oracle_linear_minibatch_2w0(B, H, N, d, int(minibatch), int(mode), _p(K), _p(Q), _p(V),
                                               _p(W0), _p(eta), _p(Z), int(threads)), "linear_minibatch_2w0")
    return Z


def linear_gradient_magnitude(K, V, W0, loss: int = L2, threads: int = 0):
    """Per-token ||G_t||_F at W0 (the gradient magnitude map), [B,H,N]."""
    K, V, W0 = map(_f64, (K, V, W0))
    B, H, N, d = K.shape
    out = np.empty((B, H, N))
    _check(_load().oracle_linear_gradient_magnitude(B, H, N, d, int(loss), _p(K), _p(V), _p(W0), _p(out),
                                                    int(threads)), "linear_gradient_magnitude")
    return out


def linear_minibatch_bwd(K, Q, V, W0, eta, dZ, minibatch: int, mode: int = FORWARD_BACKWARD_AVG,
                         threads: int = 0):
    """Gradients of sum(dZ * Z) through linear_minibatch.

    Returns (dK, dQ, dV, dW0, deta); dW0 [H,d,d] and deta [H] are summed over
    the batch and the scan directions."""
    K, Q, V, W0, eta, dZ = map(_f64, (K, Q, V, W0, eta, dZ))
    B, H, N, d = K.shape
    out = [np.empty_like(K) for _ in range(3)] + [np.empty((H, d, d)), np.empty((H,))]
    _check(_load().oracle_linear_minibatch_bwd(B, H, N, d, int(minibatch), int(mode), _p(K), _p(Q), _p(V),
                                               _p(W0), _p(eta), _p(dZ), *(_p(o) for o in out), int(threads)),
           "linear_minibatch_bwd")
    return tuple(out)


def mlp_fullbatch(K, Q, V, W1, W2, eta, threads: int = 0):
    """One full-batch L2 step of the two-layer SiLU MLP inner model
    f(k) = W2 silu(W1 k), then z = f'(q).  W1 [H,rd,d], W2 [H,d,rd].
    Returns (Z, dW1, dW2) with the gradients per slice [B,H,...]."""
    K, Q, V, W1, W2, eta = map(_f64, (K, Q, V, W1, W2, eta))
    B, H, N, d = K.shape
    hid = W1.shape[1]
    if W1.shape != (H, hid, d) or W2.shape != (H, d, hid):
        raise ValueError("W1 must be [H,rd,d] and W2 [H,d,rd]")
    Z = np.empty_like(K)
    G1 = np.empty((B, H, hid, d))
    G2 = np.empty((B, H, d, hid))
    _check(_load().oracle_mlp_fullbatch(B, H, N, d, hid, _p(K), _p(Q), _p(V), _p(W1), _p(W2), _p(eta), _p(Z),
                                        _p(G1), _p(G2), int(threads)), "mlp_fullbatch")
    return Z, G1, G2
