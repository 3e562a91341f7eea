"""GPU test of ttt_linear_fullbatch_noalloc, the entry point for callers
that cannot allocate: through the C ABI, its outputs (Z and the saved A/G)
equal those of ttt_linear_fullbatch on the same inputs bit for bit and
match the fp64 oracle, on two calls in a row (the second smaller), with
and without a saved buffer, and on a split slice (the scratch's counters
and partials) and an unsplit one."""
import pytest
import torch

import oracle
from tests.parity import TOL, banner, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(B, H, N, seed):
    inp = wl.draw(B, H, N, seed=seed, dtype="bf16", unit_rows=True, eta_fixed=None)
    d = torch.device("cuda:0")
    return {k: v.to(d) for k, v in inp.items()}


@pytest.mark.parametrize("with_saved", [False, True])
def test_noalloc_equals_workspace_entry_point(with_saved):
    import vision_test_sequence_amd as vt
    from vision_test_sequence_amd import binding as bd
    # 16 split slices of 6084 tokens, then 2 x 3 slices of 700 tokens
    for B, H, N, seed in ((8, 2, 6084, 1201), (2, 3, 700, 1202)):
        banner(f"noalloc B={B} H={H} N={N} saved={with_saved}")
        g = _inputs(B, H, N, seed)
        assert bd.plan_linear(B, H, N, with_saved=with_saved).splits > 1
        sv1 = torch.full((B, H, 2, 64, 64), float("nan"), device=g["K"].device) if with_saved else None
        sv2 = torch.full((B, H, 2, 64, 64), float("nan"), device=g["K"].device) if with_saved else None
        Z1 = vt.ttt_linear_fullbatch_noalloc(g["K"], g["Q"], g["V"], g["W0"], g["eta"], saved=sv1)
        Z2 = vt.ttt_linear_fullbatch(g["K"], g["Q"], g["V"], g["W0"], g["eta"], saved=sv2)
        torch.cuda.synchronize()
        assert torch.equal(Z1, Z2)
        if with_saved:
            assert torch.equal(sv1, sv2)
        Zr, Gr = oracle.linear_fullbatch(f64(g["K"]), f64(g["Q"]), f64(g["V"]), f64(g["W0"]), f64(g["eta"]))
        assert slice_rel_err(f64(Z1), Zr) <= TOL["bf16"]
        if with_saved:
            assert slice_rel_err(f64(sv1[:, :, 1]), Gr) <= TOL["bf16"]


def test_noalloc_unsplit_and_zero_init():
    import vision_test_sequence_amd as vt
    banner("noalloc one workgroup per slice, then W0 = 0 on split slices")
    g = _inputs(128, 2, 196, 1203)
    Z1 = vt.ttt_linear_fullbatch_noalloc(g["K"], g["Q"], g["V"], g["W0"], g["eta"])
    Z2 = vt.ttt_linear_fullbatch(g["K"], g["Q"], g["V"], g["W0"], g["eta"])
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z2)
    g = _inputs(4, 2, 3000, 1204)
    W0 = torch.zeros_like(g["W0"])
    Z1 = vt.ttt_linear_fullbatch_noalloc(g["K"], g["Q"], g["V"], W0, g["eta"])
    Z2 = vt.ttt_linear_fullbatch(g["K"], g["Q"], g["V"], W0, g["eta"])
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z2)
    Zr, _ = oracle.linear_fullbatch(f64(g["K"]), f64(g["Q"]), f64(g["V"]), f64(W0), f64(g["eta"]))
    assert slice_rel_err(f64(Z1), Zr) <= TOL["bf16"]
