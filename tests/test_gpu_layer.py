"""GPU tests of ttt_layer_fullbatch: the linear heads and the depthwise-conv
heads of one layer in one call.  Its outputs must equal, bit for bit, those
of ttt_linear_fullbatch and ttt_dwconv3x3_fullbatch on the same heads (those
two are checked against the fp64 oracle by their own tests); one slice of
each is also checked against the oracle here.  Covers the fused launch (the
1248x1248 stack: linear heads split over workgroups, one conv tile per
workgroup), shapes that fall back to two launches, an empty half, repeated
calls on one workspace, and determinism."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, banner, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(name, **kw):
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in wl.make(name, **kw).items()}
    return wl.WORKLOADS[name], g


def _split(w, g):
    lin = w.head_indices(wl.LINEAR)
    cv = w.head_indices(wl.DWCONV)
    l0, l1 = lin[0], lin[-1] + 1
    c0, c1 = cv[0], cv[-1] + 1
    assert lin == list(range(l0, l1)) and cv == list(range(c0, c1))
    return (l0, l1), (c0, c1)


def _layer(w, g, Z=None):
    import vision_test_sequence_amd as vt
    (l0, l1), (c0, c1) = _split(w, g)
    Z = torch.full_like(g["Q"], float("nan")) if Z is None else Z
    vt.ttt_layer_fullbatch(g["K"][:, l0:l1], g["Q"][:, l0:l1], g["V"][:, l0:l1],
                           g["W0"][l0:l1].contiguous(), g["eta"][l0:l1].contiguous(),
                           g["K"][:, c0:c1], g["Q"][:, c0:c1], g["V"][:, c0:c1],
                           g["w0"][c0:c1].contiguous(), g["eta"][c0:c1].contiguous(),
                           w.grid_h, w.grid_w, Zl=Z[:, l0:l1], Zc=Z[:, c0:c1])
    torch.cuda.synchronize()
    return Z


def _separate(w, g):
    import vision_test_sequence_amd as vt
    (l0, l1), (c0, c1) = _split(w, g)
    Z = torch.full_like(g["Q"], float("nan"))
    vt.ttt_linear_fullbatch(g["K"][:, l0:l1], g["Q"][:, l0:l1], g["V"][:, l0:l1],
                            g["W0"][l0:l1].contiguous(), g["eta"][l0:l1].contiguous(), Z=Z[:, l0:l1])
    vt.ttt_dwconv3x3_fullbatch(g["K"][:, c0:c1], g["Q"][:, c0:c1], g["V"][:, c0:c1],
                               g["w0"][c0:c1].contiguous(), g["eta"][c0:c1].contiguous(),
                               w.grid_h, w.grid_w, Z=Z[:, c0:c1])
    torch.cuda.synchronize()
    return Z


def _oracle_slices(w, g, Z, b):
    """Image b of every head against the fp64 oracle."""
    (l0, l1), (c0, c1) = _split(w, g)
    tol = TOL["bf16" if g["K"].dtype == torch.bfloat16 else "f32"]
    sl = lambda t, h0, h1: f64(t[b:b + 1, h0:h1])
    Zr, _ = oracle.linear_fullbatch(sl(g["K"], l0, l1), sl(g["Q"], l0, l1), sl(g["V"], l0, l1),
                                    f64(g["W0"][l0:l1]), f64(g["eta"][l0:l1]))
    assert slice_rel_err(sl(Z, l0, l1), Zr) <= tol
    Zc, _ = oracle.dwconv3x3_fullbatch(sl(g["K"], c0, c1), sl(g["Q"], c0, c1), sl(g["V"], c0, c1),
                                       f64(g["w0"][c0:c1]), f64(g["eta"][c0:c1]), w.grid_h, w.grid_w)
    assert slice_rel_err(sl(Z, c0, c1), Zc) <= tol


@pytest.mark.parametrize("name", ["vit3t_1248_bf16", "vit3t_224_bf16", "tiny_f32"])
def test_layer_equals_separate_calls(name):
    banner(f"layer {name}")
    w, g = _inputs(name)
    Z = _layer(w, g)
    Zs = _separate(w, g)
    assert not torch.isnan(Z.float()).any()
    assert torch.equal(Z, Zs)
    _oracle_slices(w, g, Z, 0)
    _oracle_slices(w, g, Z, g["K"].shape[0] - 1)


def test_layer_repeat_and_determinism():
    banner("layer repeated calls")
    w, g = _inputs("vit3t_1248_bf16")
    Z0 = _layer(w, g)
    w2, g2 = _inputs("vit3t_1248_bf16", seed_offset=5)
    Z1 = _layer(w2, g2)
    assert not torch.equal(Z0, Z1)
    for _ in range(3):
        assert torch.equal(_layer(w, g), Z0)
        assert torch.equal(_layer(w2, g2), Z1)


def test_layer_smaller_batch_after_larger():
    banner("layer B=3 after B=8")
    w, g = _inputs("vit3t_1248_bf16")
    _layer(w, g)
    g3 = {k: (v[:3].contiguous() if k in ("K", "Q", "V") else v) for k, v in g.items()}
    Z = _layer(w, g3)
    assert torch.equal(Z, _separate(w, g3))
    _oracle_slices(w, g3, Z, 2)


def test_layer_with_an_empty_half():
    import vision_test_sequence_amd as vt
    banner("layer with no conv heads / no linear heads")
    w, g = _inputs("vit3t_1248_bf16")
    Zs = _separate(w, g)
    Z = torch.full_like(g["Q"], float("nan"))
    e = g["K"][:, 2:2]
    vt.ttt_layer_fullbatch(g["K"][:, 0:2], g["Q"][:, 0:2], g["V"][:, 0:2], g["W0"][0:2].contiguous(),
                           g["eta"][0:2].contiguous(), e, e, e, g["w0"][2:2].contiguous(),
                           g["eta"][2:2].contiguous(), w.grid_h, w.grid_w, Zl=Z[:, 0:2], Zc=Z[:, 2:2])
    vt.ttt_layer_fullbatch(g["K"][:, 0:0], g["Q"][:, 0:0], g["V"][:, 0:0], g["W0"][0:0].contiguous(),
                           g["eta"][0:0].contiguous(), g["K"][:, 2:3], g["Q"][:, 2:3], g["V"][:, 2:3],
                           g["w0"][2:3].contiguous(), g["eta"][2:3].contiguous(), w.grid_h, w.grid_w,
                           Zl=Z[:, 0:0], Zc=Z[:, 2:3])
    torch.cuda.synchronize()
    assert torch.equal(Z, Zs)


def test_layer_workspace_shared_across_shapes():
    banner("layer calls of different shapes on one workspace")
    runs = [_inputs(n) for n in ("vit3t_1248_bf16", "tiny_f32", "vit3t_224_bf16", "vit3t_1248_bf16", "tiny_f32")]
    for w, g in runs:
        Z = _layer(w, g)
        assert torch.equal(Z, _separate(w, g)), w.name
