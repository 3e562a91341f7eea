"""GPU parity of ttt_dwconv3x3_fullbatch against the fp64 oracle, through
the C ABI: the conv heads of the three layer workloads, zero-init runs where
Z is all update, odd and degenerate grids, grids wide enough to need column
bands, and enough slices that one workgroup walks several tiles."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, banner, dtype_key, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _dev():
    return torch.device("cuda:0")


def _check(K, Q, V, w0, eta, gh, gw, tol=None):
    import vision_test_sequence_amd as vt
    B, H, N, d = K.shape
    saved = torch.full((B, H, d, 3, 3), float("nan"), device=K.device)
    Z = vt.ttt_dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw, saved=saved)
    torch.cuda.synchronize()
    Zr, gr = oracle.dwconv3x3_fullbatch(f64(K), f64(Q), f64(V), f64(w0), f64(eta), gh, gw)
    tol = tol or TOL[dtype_key(K)]
    ez = slice_rel_err(f64(Z), Zr)
    eg = slice_rel_err(f64(saved), gr)
    assert ez <= tol, f"Z rel err {ez:.3e} > {tol}"
    assert eg <= tol, f"g rel err {eg:.3e} > {tol}"
    return Z


def _conv_heads(inp, name):
    w = wl.WORKLOADS[name]
    hs = w.head_indices(wl.DWCONV)
    h0, h1 = hs[0], hs[-1] + 1
    d = _dev()
    return (inp["K"].to(d)[:, h0:h1], inp["Q"].to(d)[:, h0:h1], inp["V"].to(d)[:, h0:h1],
            inp["w0"][h0:h1].contiguous().to(d), inp["eta"][h0:h1].contiguous().to(d),
            w.grid_h, w.grid_w)


@pytest.mark.parametrize("name", ["tiny_f32", "vit3t_224_bf16", "vit3t_1248_bf16"])
def test_layer_conv_heads(name):
    banner(f"dwconv {name}")
    _check(*_conv_heads(wl.make(name), name))


@pytest.mark.parametrize("name", ["vit3t_224_bf16", "vit3t_1248_bf16"])
def test_zero_kernel_is_all_update(name):
    banner(f"dwconv w0=0 {name}")
    K, Q, V, w0, eta, gh, gw = _conv_heads(wl.make(name), name)
    _check(K, Q, V, torch.zeros_like(w0), eta, gh, gw)


@pytest.mark.parametrize("gh,gw", [(1, 1), (1, 17), (23, 1), (5, 7), (14, 14), (33, 9), (2, 2)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_odd_grids(gh, gw, dtype):
    banner(f"dwconv grid {gh}x{gw} {dtype}")
    inp = wl.draw(2, 2, gh * gw, seed=300 + gh * 31 + gw, dtype=dtype, eta_fixed=None)
    d = _dev()
    _check(inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["w0"].to(d), inp["eta"].to(d), gh, gw)


def test_wide_grid_uses_column_bands():
    banner("dwconv wide grid 5x300")
    inp = wl.draw(1, 1, 5 * 300, seed=401, dtype="bf16")
    d = _dev()
    _check(inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["w0"].to(d), inp["eta"].to(d), 5, 300)


def test_many_slices_walk_several_tiles():
    # more slices than resident workgroups: one workgroup per slice, which
    # walks its slice's tiles in both passes
    banner("dwconv 300 slices of 30x30")
    inp = wl.draw(100, 3, 900, seed=402, dtype="bf16", eta_fixed=None)
    d = _dev()
    _check(inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["w0"].to(d), inp["eta"].to(d), 30, 30)


def test_deterministic():
    banner("dwconv determinism")
    import vision_test_sequence_amd as vt
    K, Q, V, w0, eta, gh, gw = _conv_heads(wl.make("vit3t_1248_bf16"), "vit3t_1248_bf16")
    Z1 = vt.ttt_dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    Z2 = vt.ttt_dwconv3x3_fullbatch(K, Q, V, w0, eta, gh, gw)
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z2)


def test_workspace_shared_across_shapes():
    # calls of different shapes reuse one cached workspace: partial sums of
    # one shape must never land on the barrier counters of another
    banner("dwconv workspace shared across shapes")
    d = _dev()
    cases = [(8, 78, 78, 501), (128, 14, 14, 502), (3, 33, 20, 503), (8, 78, 78, 504), (128, 14, 14, 505)]
    for B, gh, gw, seed in cases:
        inp = wl.draw(B, 1, gh * gw, seed=seed, dtype="bf16", unit_rows=True)
        _check(inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["w0"].to(d), inp["eta"].to(d), gh, gw)


@pytest.mark.parametrize("cap", [128, 64, 24])
def test_slices_share_tiles_among_fewer_workgroups(cap):
    # fewer resident workgroups than tiles (a smaller device, forced here):
    # several consecutive tiles per workgroup and still a split exchange
    import os
    banner(f"dwconv 1248x1248 conv head, TTT_CONV_CAP={cap}")
    args = _conv_heads(wl.make("vit3t_1248_bf16"), "vit3t_1248_bf16")
    os.environ["TTT_CONV_CAP"] = str(cap)
    try:
        _check(*args)
        K, Q, V, w0, eta, gh, gw = args
        _check(K, Q, V, torch.zeros_like(w0), eta, gh, gw)
    finally:
        os.environ.pop("TTT_CONV_CAP", None)
