"""The entry points captured in one HIP graph (torch.cuda.graph) and
replayed, with eager calls and synchronisations between the replays: every
replay, and every eager call after one, must reproduce the eager outputs
bit for bit.  The exchange kernels place their splits by the XCD they run
on, so this also covers launches whose blocks start on another XCD than
block 0 -> XCD 0 (graph replays change that starting point)."""
import pytest
import torch

from tests.parity import banner, requires_gpu
from vision_test_sequence_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _ops(g, w):
    import vision_test_sequence_amd as vt

    def lin():
        vt.ttt_linear_fullbatch(g["K"][:, 0:2], g["Q"][:, 0:2], g["V"][:, 0:2], g["W0l"], g["etal"],
                                Z=g["Z"][:, 0:2])

    def conv():
        vt.ttt_dwconv3x3_fullbatch(g["K"][:, 2:3], g["Q"][:, 2:3], g["V"][:, 2:3], g["w0c"], g["etac"],
                                   w.grid_h, w.grid_w, Z=g["Z"][:, 2:3])

    def lin_saved():
        vt.ttt_linear_fullbatch(g["Ks"], g["Qs"], g["Vs"], g["W0l"], g["etal"], Z=g["Zs"], saved=g["sv"])

    def scan():
        vt.ttt_linear_minibatch_bidir(g["Ks"], g["Qs"], g["Vs"], g["W0l"], g["etal"], 16, Z=g["Zm"])

    def bwd():
        vt.ttt_linear_fullbatch_bwd(g["Ks"], g["Qs"], g["Vs"], g["W0l"], g["etal"], g["dZ"], saved=g["sv"],
                                    dK=g["dK"], dQ=g["dQ"], dV=g["dV"], dW0=g["dW0"], deta=g["deta"])

    def layer():
        vt.ttt_layer_fullbatch(g["K"][:, 0:2], g["Q"][:, 0:2], g["V"][:, 0:2], g["W0l"], g["etal"],
                               g["K"][:, 2:3], g["Q"][:, 2:3], g["V"][:, 2:3], g["w0c"], g["etac"],
                               w.grid_h, w.grid_w, Zl=g["Zy"][:, 0:2], Zc=g["Zy"][:, 2:3])

    return [lin, conv, lin_saved, scan, bwd, layer]


OUTS = ("Z", "Zs", "sv", "Zm", "dK", "dQ", "dV", "dW0", "deta", "Zy")


def test_graph_replay_matches_eager():
    banner("graph capture / replay of the entry points")
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS["vit3t_1248_bf16"]
    g = {k: v.to(dev) for k, v in wl.make("vit3t_1248_bf16").items()}
    g["W0l"] = g["W0"][0:2].contiguous()
    g["etal"] = g["eta"][0:2].contiguous()
    g["w0c"] = g["w0"][2:3].contiguous()
    g["etac"] = g["eta"][2:3].contiguous()
    g["Z"] = torch.zeros_like(g["Q"])
    g["Zy"] = torch.zeros_like(g["Q"])
    # a smaller problem for the saved-A/G forward, the scans and the backward
    s = {k: v.to(dev) for k, v in wl.make("vit3t_224_bf16").items()}
    g["Ks"], g["Qs"], g["Vs"] = (s[k][:, 0:2].contiguous() for k in ("K", "Q", "V"))
    B, _, N, d = g["Ks"].shape
    g["Zs"], g["Zm"] = torch.zeros_like(g["Qs"]), torch.zeros_like(g["Qs"])
    g["sv"] = torch.zeros((B, 2, 2, d, d), dtype=torch.float32, device=dev)
    g["dZ"] = (torch.randn(g["Qs"].shape, generator=torch.Generator().manual_seed(7)) * 0.1).to(
        dev, g["Qs"].dtype)
    for k in ("dK", "dQ", "dV"):
        g[k] = torch.zeros_like(g["Qs"])
    g["dW0"] = torch.zeros((2, d, d), dtype=torch.float32, device=dev)
    g["deta"] = torch.zeros((2,), dtype=torch.float32, device=dev)
    ops = _ops(g, w)

    def run_all():
        for op in ops:
            op()

    def clear():
        for k in OUTS:
            g[k].zero_()

    run_all()
    torch.cuda.synchronize()
    ref = {k: g[k].clone() for k in OUTS}
    for k in OUTS:
        assert not torch.isnan(ref[k].float()).any(), f"eager {k} has NaN"
    assert torch.equal(ref["Zy"], ref["Z"])  # the layer call equals the two separate calls

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()  # warm-up on a side stream, as torch asks before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):  # the warm-up stream: its workspaces exist
        run_all()
    torch.cuda.synchronize()
    for r in range(3):
        clear()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(g[k], ref[k]), f"replay {r}: {k} differs from the eager result"
        clear()
        run_all()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(g[k], ref[k]), f"eager call after replay {r}: {k} differs"
        print(f"replay {r} ok", flush=True)
