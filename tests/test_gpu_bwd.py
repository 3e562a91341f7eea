"""GPU parity of ttt_linear_fullbatch_bwd against the fp64 oracle, through
the C ABI: the finite-difference-pinned fp32 slice (B=1, H=1, N=64) at
1e-5, larger fp32 problems at 1e-5, the ViT-B 1024x1024 forward+backward
batch in bf16 (A and G saved by the forward), the recompute path (no saved
buffer) against the saved path, ragged token counts, strided views and
determinism."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, banner, dtype_key, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _dev():
    return torch.device("cuda:0")


def _head_err(got, ref):
    """||.||_inf relative error per head of an [H, ...] tensor, max over heads."""
    g = np.asarray(got, np.float64).reshape(got.shape[0], -1)
    r = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    return float(np.max(np.max(np.abs(g - r), axis=1) / np.maximum(np.max(np.abs(r), axis=1), 1e-300)))


def _vec_err(got, ref):
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    return float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300))


def _run(K, Q, V, W0, eta, dZ, use_saved=True):
    import vision_test_sequence_amd as vt
    saved = None
    if use_saved:
        B, H, N, d = K.shape
        saved = torch.empty((B, H, 2, d, d), dtype=torch.float32, device=K.device)
        vt.ttt_linear_fullbatch(K, Q, V, W0, eta, saved=saved)
    out = vt.ttt_linear_fullbatch_bwd(K, Q, V, W0, eta, dZ, saved=saved)
    torch.cuda.synchronize()
    return out


def _check(inp, use_saved=True, tol=None):
    d = _dev()
    K, Q, V, dZ = (inp[k].to(d) for k in ("K", "Q", "V", "dZ"))
    W0, eta = inp["W0"].to(d), inp["eta"].to(d)
    dK, dQ, dV, dW0, deta = _run(K, Q, V, W0, eta, dZ, use_saved)
    rK, rQ, rV, rW0, reta = oracle.linear_fullbatch_bwd(f64(K), f64(Q), f64(V), f64(W0), f64(eta),
                                                        f64(dZ))
    tol = tol or TOL[dtype_key(K)]
    errs = {"dK": slice_rel_err(f64(dK), rK), "dQ": slice_rel_err(f64(dQ), rQ),
            "dV": slice_rel_err(f64(dV), rV), "dW0": _head_err(f64(dW0), rW0),
            "deta": _vec_err(f64(deta), reta)}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"rel errs above {tol}: {bad} (all: {errs})"
    return dK, dQ, dV, dW0, deta


def test_fd_pinned_fp32_slice():
    # the slice whose oracle gradients are pinned by central differences
    banner("bwd fp32 B=1 H=1 N=64")
    _check(wl.draw(1, 1, 64, seed=1000, dtype="f32", eta_fixed=None, backward=True))


@pytest.mark.parametrize("B,H,N", [(2, 3, 300), (1, 2, 1000), (3, 1, 17), (1, 1, 1)])
def test_fp32_problems(B, H, N):
    banner(f"bwd fp32 B={B} H={H} N={N}")
    _check(wl.draw(B, H, N, seed=1100 + N, dtype="f32", eta_fixed=None, backward=True))


def test_vitb_1024_batch():
    banner("bwd vitb_1024_fwdbwd_bf16")
    _check(wl.make("vitb_1024_fwdbwd_bf16"))


@pytest.mark.parametrize("N", [1, 33, 200, 1000, 6084])
def test_ragged_bf16(N):
    banner(f"bwd bf16 N={N}")
    _check(wl.draw(2, 3, N, seed=1200 + N, dtype="bf16", eta_fixed=None, backward=True))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recompute_matches_saved(dtype):
    banner(f"bwd recompute vs saved {dtype}")
    inp = wl.draw(3, 2, 2500, seed=1300, dtype=dtype, eta_fixed=None, backward=True)
    d = _dev()
    K, Q, V, dZ = (inp[k].to(d) for k in ("K", "Q", "V", "dZ"))
    W0, eta = inp["W0"].to(d), inp["eta"].to(d)
    a = _run(K, Q, V, W0, eta, dZ, use_saved=True)
    b = _run(K, Q, V, W0, eta, dZ, use_saved=False)
    for x, y, name in zip(a, b, ("dK", "dQ", "dV", "dW0", "deta")):
        assert torch.equal(x, y), name
    _check(inp, use_saved=False)


def test_strided_views_and_shared_qk():
    banner("bwd strided, Q = K")
    B, H, N = 2, 2, 700
    inp = wl.draw(B, H, N, seed=1400, dtype="bf16", eta_fixed=None, backward=True)
    inp["Q"] = inp["K"]
    dev = _dev()
    tm = lambda t: t.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    K, V, dZ = tm(inp["K"]), tm(inp["V"]), tm(inp["dZ"])
    W0, eta = inp["W0"].to(dev), inp["eta"].to(dev)
    import vision_test_sequence_amd as vt
    dK, dQ, dV, dW0, deta = vt.ttt_linear_fullbatch_bwd(K, K, V, W0, eta, dZ)
    torch.cuda.synchronize()
    rK, rQ, rV, rW0, reta = oracle.linear_fullbatch_bwd(f64(K), f64(K), f64(V), f64(W0), f64(eta),
                                                        f64(dZ))
    tol = TOL["bf16"]
    # with Q = K the caller adds dK and dQ; each is checked on its own
    assert slice_rel_err(f64(dK), rK) <= tol
    assert slice_rel_err(f64(dQ), rQ) <= tol
    assert slice_rel_err(f64(dV), rV) <= tol
    assert _head_err(f64(dW0), rW0) <= tol
    assert _vec_err(f64(deta), reta) <= tol


def test_deterministic():
    banner("bwd determinism")
    inp = wl.draw(4, 3, 4096, seed=1500, dtype="bf16", eta_fixed=None, backward=True)
    d = _dev()
    K, Q, V, dZ = (inp[k].to(d) for k in ("K", "Q", "V", "dZ"))
    W0, eta = inp["W0"].to(d), inp["eta"].to(d)
    a = _run(K, Q, V, W0, eta, dZ)
    b = _run(K, Q, V, W0, eta, dZ)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_workspace_reuse_across_shapes():
    """bf16 pass 1 counts each slice's finished splits on the workspace's
    counter block and the last one resets it: calls of different shapes
    alternating on one workspace give the same results every time."""
    banner("bwd workspace reuse across shapes")
    d = _dev()
    sets = []
    for (B, H, N), seed in (((2, 3, 700), 1510), ((4, 3, 4096), 1511), ((1, 2, 129), 1512)):
        inp = wl.draw(B, H, N, seed=seed, dtype="bf16", eta_fixed=None, backward=True)
        sets.append([inp[k].to(d) for k in ("K", "Q", "V", "W0", "eta", "dZ")])
    first = [_run(*s) for s in sets]
    for _ in range(2):
        for s, ref in zip(sets, first):
            again = _run(*s)
            for x, y, name in zip(again, ref, ("dK", "dQ", "dV", "dW0", "deta")):
                assert torch.equal(x, y), name
    _check(dict(zip(("K", "Q", "V", "W0", "eta", "dZ"), (t.cpu() for t in sets[1]))))
