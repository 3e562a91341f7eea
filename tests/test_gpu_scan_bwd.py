"""GPU parity of ttt_linear_minibatch_bidir_bwd against the fp64 oracle
(whose scan backward is pinned by finite differences on the CPU), through
the C ABI: fp32 slices at 1e-5 over mini-batch sizes 1 .. 32 with ragged
last mini-batches in all three modes, the Vision-TTT-S 1280x1280 workload
(B=4, H=6, N=6400, b=16, both directions) in bf16 at 2e-2, and one initial
state per direction (checked through the shared-state results)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, banner, dtype_key, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _dev():
    return torch.device("cuda:0")


def _vec_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _run(g, b, mode, W0=None):
    import vision_test_sequence_amd as vt
    out = vt.ttt_linear_minibatch_bidir_bwd(g["K"], g["Q"], g["V"], g["W0"] if W0 is None else W0, g["eta"],
                                            g["dZ"], b, mode)
    torch.cuda.synchronize()
    return out


def _check(g, b, mode, tol=None):
    out = _run(g, b, mode)
    ref = oracle.linear_minibatch_bwd(*(f64(g[k]) for k in ("K", "Q", "V", "W0", "eta", "dZ")), b, mode)
    tol = tol or TOL[dtype_key(g["K"])]
    for name, got, r in zip(("dK", "dQ", "dV"), out[:3], ref[:3]):
        e = slice_rel_err(f64(got), r)
        assert e <= tol, f"{name} rel err {e:.3e} > {tol}"
    e = slice_rel_err(f64(out[3])[None], ref[3][None])
    assert e <= tol, f"dW0 rel err {e:.3e} > {tol}"
    e = _vec_err(f64(out[4]), ref[4])
    assert e <= tol, f"deta rel err {e:.3e} > {tol}"
    return out


def _draw(B, H, N, seed, dtype, unit_rows=True):
    return {k: v.to(_dev()) for k, v in wl.draw(B, H, N, seed=seed, dtype=dtype, unit_rows=unit_rows,
                                                 eta_fixed=None, backward=True).items()}


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,b", [(37, 1), (37, 5), (37, 16), (70, 32), (16, 16), (1, 4)])
def test_fp32_slices(mode, N, b):
    banner(f"scan bwd fp32 N={N} b={b} mode={mode}")
    _check(_draw(1, 2, N, 1600 + N + b + mode, "f32", unit_rows=False), b, mode)


def test_vittt_s_1280_bf16():
    banner("scan bwd bf16 vittt_s_1280 (B=4, H=6, N=6400, b=16, both directions)")
    w = wl.WORKLOADS["vittt_s_1280_bf16"]
    g = {k: v.to(_dev()) for k, v in wl.draw(w.B, w.H, w.N, seed=w.seed, dtype="bf16", unit_rows=True,
                                              backward=True).items()}
    _check(g, w.minibatch, 0)


@pytest.mark.parametrize("mode", [1, 2])
def test_bf16_single_directions(mode):
    banner(f"scan bwd bf16 N=2000 b=16 mode={mode}")
    _check(_draw(2, 3, 2000, 1610 + mode, "bf16"), 16, mode)


def test_one_initial_state_per_direction():
    banner("scan bwd with one W0 per direction")
    g = _draw(2, 2, 300, 1620, "f32")
    # equal copies: the same gradients, and dW0 split between the directions
    same = torch.stack([g["W0"], g["W0"]]).contiguous()
    a = _run(g, 16, 0, same)
    s = _run(g, 16, 0)
    for x, y in zip(a[:3], s[:3]):
        assert slice_rel_err(f64(x), f64(y)) <= 1e-5
    assert slice_rel_err(f64(a[3][0] + a[3][1])[None], f64(s[3])[None]) <= 1e-5
    # distinct copies, forward only: the forward copy's gradients, none for the other
    W1 = torch.from_numpy(np.random.default_rng(1621).standard_normal((2, 64, 64)).astype(np.float32) / 8)
    two = torch.stack([g["W0"], W1.to(_dev())]).contiguous()
    f = _run(g, 16, 1, two)
    ref = oracle.linear_minibatch_bwd(*(f64(g[k]) for k in ("K", "Q", "V", "W0", "eta", "dZ")), 16, 1)
    assert slice_rel_err(f64(f[0]), ref[0]) <= 1e-5
    assert slice_rel_err(f64(f[3][0])[None], ref[3][None]) <= 1e-5
    assert torch.count_nonzero(f[3][1]) == 0


def _vector_walks(on):
    import os
    if on:
        os.environ["TTT_SCAN_BWD_VECTOR_WALKS"] = "1"
    else:
        os.environ.pop("TTT_SCAN_BWD_VECTOR_WALKS", None)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,b", [(37, 1), (37, 5), (300, 16), (1, 4), (16, 16), (1000, 7)])
def test_bf16_matrix_core_walks(mode, N, b):
    # bf16 views take the matrix-core walks (forward states and the gradient
    # walk); checked against the oracle and against the vector walks
    banner(f"scan bwd bf16 matrix-core walks N={N} b={b} mode={mode}")
    g = _draw(2, 2, N, 1630 + N + b + mode, "bf16")
    out = _check(g, b, mode)
    try:
        _vector_walks(True)
        ref = _run(g, b, mode)
    finally:
        _vector_walks(False)
    for name, x, y in zip(("dK", "dQ", "dV"), out[:3], ref[:3]):
        assert slice_rel_err(f64(x), f64(y)) <= TOL["bf16"], name


def test_bf16_walks_with_one_initial_state_per_direction():
    banner("scan bwd bf16 walks, one W0 per direction")
    import vision_test_sequence_amd as vt
    g = _draw(2, 2, 500, 1640, "bf16")
    W1 = torch.from_numpy(np.random.default_rng(1641).standard_normal((2, 64, 64)).astype(np.float32) / 8)
    two = torch.stack([g["W0"], W1.to(_dev())]).contiguous()
    out = vt.ttt_linear_minibatch_bidir_bwd(g["K"], g["Q"], g["V"], two, g["eta"], g["dZ"], 16, 0)
    torch.cuda.synchronize()
    try:
        _vector_walks(True)
        ref = vt.ttt_linear_minibatch_bidir_bwd(g["K"], g["Q"], g["V"], two, g["eta"], g["dZ"], 16, 0)
        torch.cuda.synchronize()
    finally:
        _vector_walks(False)
    for x, y in zip(out, ref):
        assert slice_rel_err(f64(x).reshape(1, -1), f64(y).reshape(1, -1)) <= TOL["bf16"]
