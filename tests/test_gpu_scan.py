"""GPU parity of ttt_linear_minibatch_bidir against the fp64 oracle, through
the C ABI: the Vision-TTT-S 1280x1280 layer (6400 tokens, b=16, both
scans averaged), single-direction modes, ragged last chunks, small and odd
mini-batch sizes (b=1 is per-token gradient descent), sequences short
enough that every token is averaged after the scan and long enough that
most are averaged in flight, zero-init states, strided layouts with Q
aliasing K, and determinism."""
import pytest
import torch

import oracle
from tests.parity import TOL, banner, f64, requires_gpu, slice_rel_err
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

BIDIR, FWD, BWD = 0, 1, 2


def _dev():
    return torch.device("cuda:0")


def _check(K, Q, V, W0, eta, b, mode, tol=None):
    import vision_test_sequence_amd as vt
    Z = vt.ttt_linear_minibatch_bidir(K, Q, V, W0, eta, b, mode)
    torch.cuda.synchronize()
    Zr = oracle.linear_minibatch(f64(K), f64(Q), f64(V), f64(W0), f64(eta), b, mode)
    err = slice_rel_err(f64(Z), Zr)
    tol = tol or TOL["bf16"]
    assert err <= tol, f"Z rel err {err:.3e} > {tol} (b={b}, mode={mode})"
    return Z


def _on(inp):
    d = _dev()
    return (inp["K"].to(d), inp["Q"].to(d), inp["V"].to(d), inp["W0"].to(d), inp["eta"].to(d))


def test_vittt_s_1280_layer():
    banner("scan vittt_s_1280_bf16 bidir b=16")
    w = wl.WORKLOADS["vittt_s_1280_bf16"]
    _check(*_on(wl.make("vittt_s_1280_bf16")), w.minibatch, BIDIR)


@pytest.mark.parametrize("mode", [FWD, BWD])
def test_single_direction_modes(mode):
    banner(f"scan single direction mode={mode}")
    inp = wl.draw(2, 3, 2000, seed=700 + mode, dtype="bf16", unit_rows=True)
    _check(*_on(inp), 16, mode)


@pytest.mark.parametrize("N,b", [(196, 16), (196, 4), (200, 7), (17, 16), (1, 16), (5, 1),
                                 (64, 1), (2000, 16), (1000, 3), (999, 16)])
def test_ragged_and_small_minibatches(N, b):
    banner(f"scan bidir N={N} b={b}")
    inp = wl.draw(2, 2, N, seed=800 + N + 13 * b, dtype="bf16", unit_rows=True)
    _check(*_on(inp), b, BIDIR)


@pytest.mark.parametrize("mode", [BIDIR, FWD, BWD])
def test_zero_init_state(mode):
    banner(f"scan W0=0 mode={mode}")
    inp = wl.draw(2, 2, 1500, seed=900 + mode, dtype="bf16", unit_rows=True)
    K, Q, V, W0, eta = _on(inp)
    _check(K, Q, V, torch.zeros_like(W0), eta, 16, mode)


def test_varied_step_sizes():
    banner("scan eta ~ U[0.5, 2]")
    inp = wl.draw(3, 4, 1200, seed=950, dtype="bf16", unit_rows=True, eta_fixed=None)
    _check(*_on(inp), 16, BIDIR)


def test_token_major_layout_and_shared_qk():
    banner("scan strided layout, Q = K")
    B, H, N = 2, 3, 1111
    inp = wl.draw(B, H, N, seed=960, dtype="bf16", unit_rows=True)
    dev = _dev()
    Kt = inp["K"].permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    Vt = inp["V"].permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    _check(Kt, Kt, Vt, inp["W0"].to(dev), inp["eta"].to(dev), 16, BIDIR)


@pytest.mark.parametrize("mode", [BIDIR, FWD, BWD])
def test_token_major_output_with_guard_head(mode):
    """Z written into a token-major buffer with a spare head between rows:
    the outputs match the oracle and the spare head stays untouched (the
    walk's overrun and empty slots store nothing)."""
    import vision_test_sequence_amd as vt
    banner(f"scan token-major Z, mode {mode}")
    B, H, N, b = 2, 3, 203, 7
    inp = wl.draw(B, H, N, seed=961, dtype="bf16", unit_rows=True)
    dev = _dev()
    K, Q, V, W0, eta = (inp[k].to(dev) for k in ("K", "Q", "V", "W0", "eta"))
    buf = torch.full((B, N, H + 1, 64), float("nan"), dtype=K.dtype, device=dev)
    Z = buf[:, :, :H].permute(0, 2, 1, 3)
    vt.ttt_linear_minibatch_bidir(K, Q, V, W0, eta, b, mode, Z=Z)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:, :, H].float()).all()
    Zr = oracle.linear_minibatch(f64(K), f64(Q), f64(V), f64(W0), f64(eta), b, mode)
    assert slice_rel_err(f64(Z), Zr) <= TOL["bf16"]


def test_deterministic():
    banner("scan determinism")
    import vision_test_sequence_amd as vt
    K, Q, V, W0, eta = _on(wl.draw(4, 6, 6400, seed=970, dtype="bf16", unit_rows=True))
    Z1 = vt.ttt_linear_minibatch_bidir(K, Q, V, W0, eta, 16, BIDIR)
    Z2 = vt.ttt_linear_minibatch_bidir(K, Q, V, W0, eta, 16, BIDIR)
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z2)


def test_fp32_inputs_are_rejected():
    banner("scan fp32 -> unsupported")
    import vision_test_sequence_amd as vt
    from vision_test_sequence_amd.binding import TTTError
    K, Q, V, W0, eta = _on(wl.draw(1, 1, 64, seed=980, dtype="f32"))
    with pytest.raises(TTTError):
        vt.ttt_linear_minibatch_bidir(K, Q, V, W0, eta, 16, BIDIR)


def test_workspace_shared_across_shapes():
    # calls of different shapes reuse one cached workspace: the empty-slot
    # rows it keeps must stay zero whatever an earlier call stored
    banner("scan workspace shared across shapes")
    for B, H, N, b, seed in [(4, 6, 6400, 16, 990), (2, 3, 196, 4, 991), (2, 2, 2000, 16, 992),
                             (1, 1, 37, 5, 993), (4, 6, 6400, 16, 994), (3, 1, 300, 7, 995)]:
        _check(*_on(wl.draw(B, H, N, seed=seed, dtype="bf16", unit_rows=True)), b, BIDIR)
