"""GPU parity of the inner-training variants against the fp64 oracle (whose
variants are pinned on the CPU), through the C ABI:
  * the dot-product loss in the full-batch linear step (the G-exchange,
    resident-with-saved and streaming kernels), its backward, the depthwise
    step and its backward, and the fused layer;
  * several full-batch steps (epochs) under both losses;
  * one initial state per scan direction, in all three scan modes;
  * the gradient magnitude map under both losses;
  * the combinations an operation does not take are rejected.
fp32 cases at 1e-5, bf16 at 2e-2 (per-slice inf-norm relative error)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, banner, dtype_key, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import binding as bd
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]
DOT, L2 = bd.LOSS_DOT, bd.LOSS_L2


def _dev():
    return torch.device("cuda:0")


def _on(inp):
    return {k: v.to(_dev()) for k, v in inp.items()}


def _vec_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _stack_linear():
    g = _on(wl.make("vit3t_1248_bf16"))
    return g["K"][:, 0:2], g["Q"][:, 0:2], g["V"][:, 0:2], g["W0"][0:2].contiguous(), g["eta"][0:2].contiguous()


# ------------------------------------------------------------ dot-product loss
@pytest.mark.parametrize("w0_zero", [False, True])
def test_dot_loss_linear_stack_gx(w0_zero):
    import vision_test_sequence_amd as vt
    banner(f"variants: dot loss, 1248 linear heads (G exchange), W0=0: {w0_zero}")
    K, Q, V, W0, eta = _stack_linear()
    if w0_zero:
        W0 = torch.zeros_like(W0)
    assert bd.plan_linear(8, 2, 6084).kernel == bd.KERNEL_LIN_RESIDENT_GX
    Z = vt.ttt_linear_fullbatch(K, Q, V, W0, eta, loss=DOT)
    torch.cuda.synchronize()
    Zr, _ = oracle.linear_fullbatch_ex(f64(K), f64(Q), f64(V), f64(W0), f64(eta), oracle.DOT, 1)
    assert slice_rel_err(f64(Z), Zr) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,B,H,N", [("f32", 2, 2, 777), ("f32", 1, 1, 20000), ("bf16", 3, 2, 6084),
                                         ("bf16", 1, 2, 40000)])
def test_dot_loss_linear_with_saved(dtype, B, H, N):
    import vision_test_sequence_amd as vt
    banner(f"variants: dot loss linear {dtype} B={B} H={H} N={N} with saved")
    g = _on(wl.draw(B, H, N, seed=1400 + N, dtype=dtype, eta_fixed=None))
    saved = torch.full((B, H, 2, 64, 64), float("nan"), device=_dev())
    Z = vt.ttt_linear_fullbatch(g["K"], g["Q"], g["V"], g["W0"], g["eta"], saved=saved, loss=DOT)
    Z2 = vt.ttt_linear_fullbatch(g["K"], g["Q"], g["V"], g["W0"], g["eta"], loss=DOT)
    torch.cuda.synchronize()
    args = [f64(g[k]) for k in ("K", "Q", "V", "W0", "eta")]
    Zr, Wr = oracle.linear_fullbatch_ex(*args, oracle.DOT, 1)
    tol = TOL[dtype]
    assert slice_rel_err(f64(Z), Zr) <= tol
    assert slice_rel_err(f64(Z2), Zr) <= tol
    Gr = (args[3][None] - Wr) / args[4][None, :, None, None]  # G = (W0 - W1) / eta
    assert slice_rel_err(f64(saved[:, :, 1]), Gr) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dot_loss_linear_backward(dtype):
    import vision_test_sequence_amd as vt
    banner(f"variants: dot loss linear backward {dtype}")
    B, H, N = (1, 1, 64) if dtype == "f32" else (4, 3, 4096)
    g = _on(wl.draw(B, H, N, seed=1410, dtype=dtype, eta_fixed=None, backward=True))
    out = vt.ttt_linear_fullbatch_bwd(g["K"], g["Q"], g["V"], g["W0"], g["eta"], g["dZ"], loss=DOT)
    torch.cuda.synchronize()
    ref = oracle.linear_fullbatch_bwd_ex(*(f64(g[k]) for k in ("K", "Q", "V", "W0", "eta", "dZ")), oracle.DOT)
    tol = TOL[dtype]
    for got, r in zip(out[:3], ref[:3]):
        assert slice_rel_err(f64(got), r) <= tol
    assert slice_rel_err(f64(out[3])[None], ref[3][None]) <= tol
    assert _vec_err(f64(out[4]), ref[4]) <= tol


@pytest.mark.parametrize("dtype,B,H,gh,gw", [("f32", 2, 2, 14, 14), ("bf16", 8, 1, 78, 78), ("bf16", 3, 2, 5, 300)])
def test_dot_loss_conv(dtype, B, H, gh, gw):
    import vision_test_sequence_amd as vt
    banner(f"variants: dot loss dwconv {dtype} {B}x{H} {gh}x{gw}")
    g = _on(wl.draw(B, H, gh * gw, seed=1420 + gw, dtype=dtype, eta_fixed=None, backward=True))
    saved = torch.full((B, H, 64, 3, 3), float("nan"), device=_dev())
    Z = vt.ttt_dwconv3x3_fullbatch(g["K"], g["Q"], g["V"], g["w0"], g["eta"], gh, gw, saved=saved, loss=DOT)
    bw = vt.ttt_dwconv3x3_fullbatch_bwd(g["K"], g["Q"], g["V"], g["w0"], g["eta"], g["dZ"], gh, gw, loss=DOT)
    torch.cuda.synchronize()
    args = [f64(g[k]) for k in ("K", "Q", "V", "w0", "eta")]
    Zr, gr = oracle.dwconv3x3_fullbatch_ex(*args, gh, gw, oracle.DOT)
    tol = TOL[dtype]
    assert slice_rel_err(f64(Z), Zr) <= tol
    assert slice_rel_err(f64(saved), gr) <= tol
    ref = oracle.dwconv3x3_fullbatch_bwd_ex(*args, f64(g["dZ"]), gh, gw, oracle.DOT)
    for got, r in zip(bw[:3], ref[:3]):
        assert slice_rel_err(f64(got), r) <= tol
    assert slice_rel_err(f64(bw[3])[None], ref[3][None]) <= tol
    assert _vec_err(f64(bw[4]), ref[4]) <= tol


def test_dot_loss_fused_layer():
    import vision_test_sequence_amd as vt
    banner("variants: dot loss, fused 1248x1248 layer")
    g = _on(wl.make("vit3t_1248_bf16", seed_offset=7))
    assert bd.plan_layer_fused((8, 2, 6084), (8, 1, 78, 78))
    Z = torch.full_like(g["Q"], float("nan"))
    lin = (g["K"][:, 0:2], g["Q"][:, 0:2], g["V"][:, 0:2], g["W0"][0:2].contiguous(), g["eta"][0:2].contiguous())
    cv = (g["K"][:, 2:3], g["Q"][:, 2:3], g["V"][:, 2:3], g["w0"][2:3].contiguous(), g["eta"][2:3].contiguous())
    vt.ttt_layer_fullbatch(*lin, *cv, 78, 78, Zl=Z[:, 0:2], Zc=Z[:, 2:3], loss=DOT)
    Zs = torch.full_like(Z, float("nan"))
    vt.ttt_linear_fullbatch(*lin, Z=Zs[:, 0:2], loss=DOT)
    vt.ttt_dwconv3x3_fullbatch(*cv, 78, 78, Z=Zs[:, 2:3], loss=DOT)
    torch.cuda.synchronize()
    assert torch.equal(Z, Zs)
    Zr, _ = oracle.linear_fullbatch_ex(*(f64(t) for t in lin), oracle.DOT, 1)
    assert slice_rel_err(f64(Z[:, 0:2]), Zr) <= TOL["bf16"]
    Zcr, _ = oracle.dwconv3x3_fullbatch_ex(*(f64(t) for t in cv), 78, 78, oracle.DOT)
    assert slice_rel_err(f64(Z[:, 2:3]), Zcr) <= TOL["bf16"]


# ------------------------------------------------------------ epochs
@pytest.mark.parametrize("loss", [L2, DOT])
@pytest.mark.parametrize("dtype,B,H,N,E", [("f32", 2, 2, 500, 3), ("f32", 1, 1, 20000, 2), ("bf16", 8, 2, 6084, 4)])
def test_several_full_batch_steps(loss, dtype, B, H, N, E):
    import vision_test_sequence_amd as vt
    banner(f"variants: {E} full-batch steps loss={loss} {dtype} B={B} H={H} N={N}")
    if dtype == "bf16":
        K, Q, V, W0, eta = _stack_linear()
        eta = torch.tensor([0.7, 1.6], device=_dev())
    else:
        g = _on(wl.draw(B, H, N, seed=1430 + N, dtype=dtype, eta_fixed=None))
        K, Q, V, W0, eta = g["K"], g["Q"], g["V"], g["W0"], g["eta"]
    Z = vt.ttt_linear_fullbatch(K, Q, V, W0, eta, loss=loss, steps=E)
    torch.cuda.synchronize()
    Zr, _ = oracle.linear_fullbatch_ex(f64(K), f64(Q), f64(V), f64(W0), f64(eta), loss, E)
    assert slice_rel_err(f64(Z), Zr) <= TOL[dtype]
    # more steps move the output: the test would see a step count ignored
    Z1, _ = oracle.linear_fullbatch_ex(f64(K), f64(Q), f64(V), f64(W0), f64(eta), loss, 1)
    assert slice_rel_err(Z1, Zr) > 3 * TOL[dtype]


@pytest.mark.parametrize("E", [2, 3])
@pytest.mark.parametrize("case", ["w0_zero", "eta_large", "ragged"])
def test_steps_inside_one_exchange_launch(monkeypatch, case, E):
    """Several steps run inside the G-exchange kernel (each split keeps A_s and
    C_s; one more exchange round per step) when the plan takes it: every
    slice against the oracle with inputs where the update dominates Z and the
    W_k A_s term of the later steps matters (W0 = 0, or eta large), against
    the three-launch path, and bit for bit on a repeat."""
    import vision_test_sequence_amd as vt
    banner(f"variants: {E} steps in one G-exchange launch, {case}")
    if case == "ragged":
        g = _on(wl.draw(3, 2, 5003, seed=1460 + E, dtype="bf16", unit_rows=True))
        K, Q, V, W0 = g["K"], g["Q"], g["V"], g["W0"]
        eta = torch.tensor([4.0, 9.0], device=_dev())
    else:
        K, Q, V, W0, eta = _stack_linear()
        if case == "w0_zero":
            W0 = torch.zeros_like(W0)
            eta = torch.tensor(np.random.default_rng(90 + E).uniform(0.5, 2.0, 2), dtype=torch.float32,
                               device=_dev())
        else:
            eta = torch.tensor([8.0, 16.0], device=_dev())
    B, H, N = K.shape[0], K.shape[1], K.shape[2]
    assert bd.plan_linear(B, H, N, steps=E).fused == 1
    Z = vt.ttt_linear_fullbatch(K, Q, V, W0, eta, steps=E)
    Z2 = vt.ttt_linear_fullbatch(K, Q, V, W0, eta, steps=E)
    torch.cuda.synchronize()
    assert torch.equal(Z, Z2)
    Zr, _ = oracle.linear_fullbatch_ex(f64(K), f64(Q), f64(V), f64(W0), f64(eta), L2, E)
    assert slice_rel_err(f64(Z), Zr) <= TOL["bf16"]
    # the last step counts: one step fewer is far from the result
    Zp, _ = oracle.linear_fullbatch_ex(f64(K), f64(Q), f64(V), f64(W0), f64(eta), L2, E - 1)
    assert slice_rel_err(Zp, Zr) > 3 * TOL["bf16"]
    monkeypatch.setenv("TTT_SPLIT_STEPS", "1")
    assert bd.plan_linear(B, H, N, steps=E).fused == 0
    Zs = vt.ttt_linear_fullbatch(K, Q, V, W0, eta, steps=E)
    torch.cuda.synchronize()
    assert slice_rel_err(f64(Zs), Zr) <= TOL["bf16"]
    assert slice_rel_err(f64(Z), f64(Zs)) <= TOL["bf16"]


# ------------------------------------------------------------ per-direction W0
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,b", [(2000, 16), (203, 7)])
def test_scan_initial_state_per_direction(mode, N, b):
    import vision_test_sequence_amd as vt
    banner(f"variants: scan W0 per direction mode={mode} N={N} b={b}")
    g = _on(wl.draw(2, 3, N, seed=1440 + N + mode, dtype="bf16", unit_rows=True))
    W1 = torch.from_numpy(np.random.default_rng(1441).standard_normal((3, 64, 64)).astype(np.float32) / 8.0)
    W0two = torch.stack([g["W0"], W1.to(_dev())]).contiguous()
    Z = vt.ttt_linear_minibatch_bidir(g["K"], g["Q"], g["V"], W0two, g["eta"], b, mode)
    torch.cuda.synchronize()
    Zr = oracle.linear_minibatch_2w0(f64(g["K"]), f64(g["Q"]), f64(g["V"]), f64(W0two), f64(g["eta"]), b, mode)
    assert slice_rel_err(f64(Z), Zr) <= TOL["bf16"]


# ------------------------------------------------------------ gradient magnitude map
@pytest.mark.parametrize("loss", [L2, DOT])
@pytest.mark.parametrize("dtype,B,H,N", [("f32", 2, 3, 777), ("f32", 1, 1, 1), ("bf16", 8, 2, 6084), ("bf16", 3, 1, 17)])
def test_gradient_magnitude_map(loss, dtype, B, H, N):
    import vision_test_sequence_amd as vt
    banner(f"variants: gradient magnitude map loss={loss} {dtype} B={B} H={H} N={N}")
    if (dtype, N) == ("bf16", 6084):
        K, _, V, W0, _ = _stack_linear()
    else:
        g = _on(wl.draw(B, H, N, seed=1450 + N, dtype=dtype))
        K, V, W0 = g["K"], g["V"], g["W0"]
    m = vt.ttt_linear_gradient_magnitude(K, V, W0, loss=loss)
    torch.cuda.synchronize()
    ref = oracle.linear_gradient_magnitude(f64(K), f64(V), f64(W0), loss)
    assert slice_rel_err(m.cpu().numpy().astype(np.float64)[..., None], ref[..., None]) <= TOL[dtype]


# ------------------------------------------------------------ rejections
def test_unsupported_combinations_are_rejected():
    import vision_test_sequence_amd as vt
    banner("variants: rejected combinations")
    g = _on(wl.draw(1, 2, 196, seed=1460, dtype="bf16"))
    K, Q, V, W0, eta, w0 = g["K"], g["Q"], g["V"], g["W0"], g["eta"], g["w0"]
    with pytest.raises(bd.TTTError, match="UNSUPPORTED"):
        vt.ttt_linear_fullbatch(K, Q, V, W0, eta, saved=torch.empty((1, 2, 2, 64, 64), device=_dev()), steps=2)
    with pytest.raises(bd.TTTError, match="UNSUPPORTED"):
        p = bd.problem(K, grid=(14, 14), steps=2)
        st = bd.lib().ttt_dwconv3x3_fullbatch(bd.ctypes.byref(p), bd.view(K), bd.view(Q), bd.view(V), w0.data_ptr(),
                                              eta.data_ptr(), bd.view(torch.empty_like(K)), None, None, 0, None)
        bd._check(st, "ttt_dwconv3x3_fullbatch")
    with pytest.raises(bd.TTTError, match="UNSUPPORTED"):
        p = bd.problem(K, minibatch=16, loss=DOT)
        st = bd.lib().ttt_linear_minibatch_bidir(bd.ctypes.byref(p), bd.view(K), bd.view(Q), bd.view(V),
                                                 W0.data_ptr(), eta.data_ptr(), bd.view(torch.empty_like(K)),
                                                 None, 0, None)
        bd._check(st, "ttt_linear_minibatch_bidir")
