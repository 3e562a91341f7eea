"""GPU parity of ttt_linear_fullbatch against the fp64 oracle, through the
C ABI.  Covers the tiny fp32 layer, the 224x224 ViT3-T batch, the
1248x1248 stack (split over many workgroups per slice), zero-init runs
where Z is all update, ragged token counts, strided/sub-range views,
shared Q/K, determinism, workspace reuse and output guard bands."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, banner, dtype_key, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _dev():
    return torch.device("cuda:0")


def _run(K, Q, V, W0, eta, with_saved=True):
    import vision_test_sequence_amd as vt
    B, H, N, d = K.shape
    saved = torch.full((B, H, 2, d, d), float("nan"), device=K.device) if with_saved else None
    Z = vt.ttt_linear_fullbatch(K, Q, V, W0, eta, saved=saved)
    torch.cuda.synchronize()
    return Z, saved


def _check(K, Q, V, W0, eta, tol=None, check_saved=True):
    Z, saved = _run(K, Q, V, W0, eta, with_saved=check_saved)
    Kd, Qd, Vd = f64(K), f64(Q), f64(V)
    Zr, Gr = oracle.linear_fullbatch(Kd, Qd, Vd, f64(W0), f64(eta))
    tol = tol or TOL[dtype_key(K)]
    ez = slice_rel_err(f64(Z), Zr)
    assert ez <= tol, f"Z rel err {ez:.3e} > {tol}"
    if check_saved:
        Ar = np.einsum("bhnc,bhne->bhce", Kd, Kd)
        eA = slice_rel_err(f64(saved[:, :, 0]), Ar)
        eG = slice_rel_err(f64(saved[:, :, 1]), Gr)
        assert eA <= tol, f"A rel err {eA:.3e}"
        assert eG <= tol, f"G rel err {eG:.3e}"
    return Z


def _head_slice(inp, heads):
    """Views of the linear heads of a mixed layer (pointer offset + strides)."""
    h0, h1 = heads[0], heads[-1] + 1
    d = _dev()
    K = inp["K"].to(d)[:, h0:h1]
    Q = inp["Q"].to(d)[:, h0:h1]
    V = inp["V"].to(d)[:, h0:h1]
    W0 = inp["W0"][h0:h1].contiguous().to(d)
    eta = inp["eta"][h0:h1].contiguous().to(d)
    return K, Q, V, W0, eta


def test_tiny_fp32_layer_linear_head():
    banner("linear tiny_f32 head 0")
    inp = wl.make("tiny_f32")
    _check(*_head_slice(inp, [0]))


def test_vit3t_224_batch_linear_heads():
    banner("linear vit3t_224_bf16 heads 0-1")
    inp = wl.make("vit3t_224_bf16")
    _check(*_head_slice(inp, [0, 1]))


def test_vit3t_1248_stack_linear_heads():
    banner("linear vit3t_1248_bf16 heads 0-1")
    inp = wl.make("vit3t_1248_bf16")
    _check(*_head_slice(inp, [0, 1]))


@pytest.mark.parametrize("name", ["vit3t_224_bf16", "vit3t_1248_bf16"])
def test_zero_init_is_all_update(name):
    # W0 = 0: Z is entirely the update term (linear attention), so the
    # Z-only check cannot be passed by an identity-like output.
    banner(f"linear W0=0 {name}")
    inp = wl.make(name)
    K, Q, V, W0, eta = _head_slice(inp, [0, 1])
    _check(K, Q, V, torch.zeros_like(W0), eta)


@pytest.mark.parametrize("N", [1, 15, 16, 17, 129, 200, 1000, 4099])
def test_ragged_token_counts_fp32(N):
    banner(f"linear ragged fp32 N={N}")
    inp = wl.draw(3, 1, N, seed=100 + N, dtype="f32", eta_fixed=None)
    d = _dev()
    _check(inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["W0"].to(d), inp["eta"].to(d))


@pytest.mark.parametrize("N", [1, 17, 300, 2500, 6084])
def test_ragged_token_counts_bf16(N):
    banner(f"linear ragged bf16 N={N}")
    inp = wl.draw(2, 5, N, seed=200 + N, dtype="bf16", unit_rows=True)
    d = _dev()
    _check(inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["W0"].to(d), inp["eta"].to(d))


def test_token_major_layout_and_shared_qk():
    # [B, N, H, d] storage viewed as [B, H, N, d]; Q aliases K.
    banner("linear strided layout, Q = K")
    B, H, N, d = 2, 3, 777, 64
    inp = wl.draw(B, H, N, seed=7, dtype="bf16")
    dev = _dev()
    Kt = inp["K"].permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    Vt = inp["V"].permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    assert Kt.stride(2) == H * d
    _check(Kt, Kt, Vt, inp["W0"].to(dev), inp["eta"].to(dev))


def test_deterministic_and_workspace_reuse():
    banner("linear determinism / workspace reuse")
    inp = wl.make("vit3t_1248_bf16")
    K, Q, V, W0, eta = _head_slice(inp, [0, 1])
    Z1, _ = _run(K, Q, V, W0, eta)
    # a different problem on the same (cached) workspace in between
    small = wl.draw(1, 1, 5000, seed=9, dtype="bf16")
    d = _dev()
    _check(small["K"].to(d), small["Q"].to(d), small["V"].to(d), small["W0"].to(d),
           small["eta"].to(d))
    Z2, _ = _run(K, Q, V, W0, eta)
    assert torch.equal(Z1, Z2)


def test_output_guard_bands_untouched():
    banner("linear guard bands")
    B, H, N, d = 2, 2, 333, 64
    inp = wl.draw(B, H, N, seed=11, dtype="bf16")
    dev = _dev()
    import vision_test_sequence_amd as vt
    # Z is the middle of a padded buffer: rows padded to 80 channels and a
    # whole spare head on each side
    big = torch.full((B, H + 2, N, 80), float("nan"), dtype=torch.bfloat16, device=dev)
    Z = big[:, 1:H + 1, :, :d]
    K, Q, V = (inp[k].to(dev) for k in "KQV")
    vt.ttt_linear_fullbatch(K, Q, V, inp["W0"].to(dev), inp["eta"].to(dev), Z=Z)
    torch.cuda.synchronize()
    assert torch.isnan(big[:, 0]).all() and torch.isnan(big[:, H + 1]).all()
    assert torch.isnan(big[:, 1:H + 1, :, d:]).all()
    Zr, _ = oracle.linear_fullbatch(f64(K), f64(Q), f64(V), f64(inp["W0"]), f64(inp["eta"]))
    assert slice_rel_err(f64(Z), Zr) <= TOL["bf16"]


def test_nan_stays_in_its_slice():
    banner("linear NaN containment")
    B, H, N, d = 2, 2, 500, 64
    inp = wl.draw(B, H, N, seed=12, dtype="bf16")
    dev = _dev()
    K, Q, V = (inp[k].clone().to(dev) for k in "KQV")
    V[1, 0, 123, 5] = float("nan")
    import vision_test_sequence_amd as vt
    Z = vt.ttt_linear_fullbatch(K, Q, V, inp["W0"].to(dev), inp["eta"].to(dev))
    torch.cuda.synchronize()
    assert torch.isnan(Z[1, 0]).any()
    for b, h in [(0, 0), (0, 1), (1, 1)]:
        assert torch.isfinite(Z[b, h]).all()


def test_workspace_shared_across_shapes():
    banner("linear workspace shared across shapes")
    d = _dev()
    for B, H, N, seed in [(8, 2, 6084, 601), (3, 7, 1000, 602), (16, 1, 4096, 603), (8, 2, 6084, 604),
                          (1, 1, 300, 605), (3, 7, 1000, 606)]:
        inp = wl.draw(B, H, N, seed=seed, dtype="bf16", unit_rows=True)
        _check(inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["W0"].to(d), inp["eta"].to(d))
