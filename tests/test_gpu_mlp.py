"""GPU parity of ttt_mlp_fullbatch (two-layer SiLU MLP inner model, one
full-batch L2 step, then applied to Q) against the fp64 oracle, whose
gradients are pinned to torch autograd and finite differences on the CPU.

bf16 views at the bf16 bar (2e-2 of each slice's largest |Z|): every width
r = 1..4 over ragged token counts (one token, fewer than a 64-token step,
ragged last steps and splits), an update-dominated case (eta large enough
that the gradient terms outweigh W1 and W2 in Z), strided head views, and
the 1248x1248 stack shape (B=8, H=3, N=6084) at width 4d with the oracle on
three of its slices."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL, banner, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _dev():
    return torch.device("cuda:0")


def _inputs(B, H, N, hid, seed, eta=None, unit_rows=False):
    g = wl.draw(B, H, N, seed=seed, dtype="bf16", unit_rows=unit_rows, eta_fixed=None)
    g.update(wl.draw_mlp_weights(H, hid, seed=seed + 1))
    if eta is not None:
        g["eta"] = torch.full((H,), float(eta), dtype=torch.float32)
    return g


def _run(g, Z=None):
    import vision_test_sequence_amd as vt
    d = {k: g[k].to(_dev()) for k in ("K", "Q", "V", "W1", "W2", "eta")}
    out = vt.ttt_mlp_fullbatch(d["K"], d["Q"], d["V"], d["W1"], d["W2"], d["eta"], Z=Z)
    torch.cuda.synchronize()
    return out


def _ref(g):
    return oracle.mlp_fullbatch(*(f64(g[k]) for k in ("K", "Q", "V", "W1", "W2", "eta")))


@pytest.mark.parametrize("hid", [64, 128, 192, 256])
@pytest.mark.parametrize("N", [1, 37, 64, 300, 1000])
def test_widths_and_ragged_token_counts(hid, N):
    banner(f"mlp bf16 hid={hid} N={N}")
    g = _inputs(2, 3, N, hid, 1700 + hid + N)
    Z = _run(g)
    Zr, _, _ = _ref(g)
    e = slice_rel_err(f64(Z), Zr)
    assert e <= TOL["bf16"], f"Z rel err {e:.3e}"


@pytest.mark.parametrize("hid", [64, 256])
def test_update_dominated(hid):
    banner(f"mlp bf16 update-dominated hid={hid}")
    g = _inputs(2, 2, 700, hid, 1750 + hid, eta=40.0)
    Zr, G1, G2 = _ref(g)
    # the gradient terms outweigh the initial weights
    W1, W2 = f64(g["W1"]), f64(g["W2"])
    assert np.abs(40.0 * G2).max() > 1.2 * np.abs(W2).max()
    assert np.abs(40.0 * G1).max() > 0.8 * np.abs(W1).max()
    Z0 = oracle.mlp_fullbatch(*(f64(g[k]) for k in ("K", "Q", "V", "W1", "W2")), np.zeros(2))[0]
    assert slice_rel_err(Z0, Zr) > 0.5                  # Z is not the untrained model's
    Z = _run(g)
    e = slice_rel_err(f64(Z), Zr)
    assert e <= TOL["bf16"], f"Z rel err {e:.3e}"


def test_strided_head_views():
    banner("mlp bf16 strided views")
    B, H, N, hid = 2, 3, 250, 128
    g = _inputs(B, H, N, hid, 1760)
    # K, Q, V as head slices of one packed [B, N, 3H, 64] tensor; Z likewise
    packed = torch.stack([g["K"], g["Q"], g["V"]], 2).permute(0, 3, 2, 1, 4).reshape(B, N, 3 * H, 64).to(_dev())
    view = lambda i: packed[:, :, i * H:(i + 1) * H].permute(0, 2, 1, 3)
    Zbuf = torch.empty((B, N, 2 * H, 64), dtype=torch.bfloat16, device=_dev())
    Z = Zbuf[:, :, H:].permute(0, 2, 1, 3)
    import vision_test_sequence_amd as vt
    vt.ttt_mlp_fullbatch(view(0), view(1), view(2), g["W1"].to(_dev()), g["W2"].to(_dev()),
                         g["eta"].to(_dev()), Z=Z)
    torch.cuda.synchronize()
    e = slice_rel_err(f64(Z), _ref(g)[0])
    assert e <= TOL["bf16"], f"Z rel err {e:.3e}"


def test_repeatable():
    banner("mlp bf16 repeat")
    g = _inputs(2, 2, 900, 192, 1770)
    a = _run(g)
    b = _run(g)
    assert torch.equal(a, b)                          # fixed-order sums


def test_1248_stack_width_4():
    banner("mlp bf16 1248x1248 stack (B=8, H=3, N=6084), hidden 256")
    w = wl.WORKLOADS["vit3t_1248_bf16"]
    g = wl.draw(w.B, w.H, w.N, seed=w.seed, dtype="bf16", unit_rows=True, eta_fixed=None)
    g.update(wl.draw_mlp_weights(w.H, 256, seed=w.seed + 1))
    Z = f64(_run(g))
    for b, h in ((0, 0), (3, 1), (7, 2)):
        sub = {k: g[k][b:b + 1, h:h + 1] for k in ("K", "Q", "V")}
        sub.update(W1=g["W1"][h:h + 1], W2=g["W2"][h:h + 1], eta=g["eta"][h:h + 1])
        e = slice_rel_err(Z[b:b + 1, h:h + 1], _ref(sub)[0])
        assert e <= TOL["bf16"], f"slice ({b},{h}) Z rel err {e:.3e}"
