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


def test_graph_replay_of_the_other_entry_points():
    # the conv and scan backwards (the scan's matrix-core walks, both with
    # coinciding and with differing direction mini-batches), the MLP inner
    # model, the gradient magnitude map, two full-batch steps, the dot loss,
    # a ragged-mini-batch scan and a chunk-parallel one, captured and replayed
    import vision_test_sequence_amd as vt
    banner("graph capture / replay of the backward, MLP and variant entry points")
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS["vit3t_1248_bf16"]
    big = {k: v.to(dev) for k, v in wl.make("vit3t_1248_bf16").items()}
    g = {}
    K, Q, V = (big[k][:, 2:3].contiguous() for k in ("K", "Q", "V"))
    g["w0c"] = big["w0"][2:3].contiguous()
    g["etac"] = big["eta"][2:3].contiguous()
    g["dZc"] = (torch.randn(Q.shape, generator=torch.Generator().manual_seed(11)) * 0.1).to(dev, Q.dtype)
    s = {k: v.to(dev) for k, v in wl.draw(2, 3, 300, seed=1700, dtype="bf16", unit_rows=True,
                                           backward=True).items()}
    mw = {k: v.to(dev) for k, v in wl.draw_mlp_weights(3, 128, seed=1701).items()}
    one = {k: v.to(dev) for k, v in wl.draw(1, 2, 6400, seed=1702, dtype="bf16", unit_rows=True).items()}
    z = lambda t: torch.zeros_like(t)
    outs = {
        "cK": z(K), "cQ": z(Q), "cV": z(V), "cw0": torch.zeros((1, 64, 3, 3), device=dev),
        "ceta": torch.zeros((1,), device=dev),
        "sK": z(s["K"]), "sQ": z(s["Q"]), "sV": z(s["V"]), "sW0": z(s["W0"]), "seta": z(s["eta"]),
        "rK": z(s["K"]), "rQ": z(s["Q"]), "rV": z(s["V"]), "rW0": z(s["W0"]), "reta": z(s["eta"]),
        "mZ": z(s["Q"]), "gmm": torch.zeros(s["K"].shape[:3], device=dev), "eZ": z(s["Q"]),
        "dZl": z(s["Q"]), "rgZ": z(s["Q"]), "cpZ": z(one["Q"]),
    }

    def conv_bwd():
        vt.ttt_dwconv3x3_fullbatch_bwd(K, Q, V, g["w0c"], g["etac"], g["dZc"], w.grid_h, w.grid_w,
                                       dK=outs["cK"], dQ=outs["cQ"], dV=outs["cV"], dw0=outs["cw0"],
                                       deta=outs["ceta"])

    def scan_bwd():  # N = 300 = 18 x 16 + 12: the directions' mini-batches differ
        vt.ttt_linear_minibatch_bidir_bwd(s["K"], s["Q"], s["V"], s["W0"], s["eta"], s["dZ"], 16, 0,
                                          dK=outs["sK"], dQ=outs["sQ"], dV=outs["sV"], dW0=outs["sW0"],
                                          deta=outs["seta"])

    def scan_bwd_even():  # b = 15 divides N: one workgroup covers both directions
        vt.ttt_linear_minibatch_bidir_bwd(s["K"], s["Q"], s["V"], s["W0"], s["eta"], s["dZ"], 15, 0,
                                          dK=outs["rK"], dQ=outs["rQ"], dV=outs["rV"], dW0=outs["rW0"],
                                          deta=outs["reta"])

    def mlp():
        vt.ttt_mlp_fullbatch(s["K"], s["Q"], s["V"], mw["W1"], mw["W2"], s["eta"], Z=outs["mZ"])

    def gmm():
        vt.ttt_linear_gradient_magnitude(s["K"], s["V"], s["W0"], out=outs["gmm"])

    def epochs():
        vt.ttt_linear_fullbatch(s["K"], s["Q"], s["V"], s["W0"], s["eta"], Z=outs["eZ"], steps=2)

    def dot():
        vt.ttt_linear_fullbatch(s["K"], s["Q"], s["V"], s["W0"], s["eta"], Z=outs["dZl"], loss=vt.LOSS_DOT)

    def ragged_scan():
        vt.ttt_linear_minibatch_bidir(s["K"], s["Q"], s["V"], s["W0"], s["eta"], 20, Z=outs["rgZ"])

    def chunk_parallel_scan():  # one image: the planner cuts the chains into segments
        vt.ttt_linear_minibatch_bidir(one["K"], one["Q"], one["V"], one["W0"], one["eta"], 16, Z=outs["cpZ"])

    ops = [conv_bwd, scan_bwd, scan_bwd_even, mlp, gmm, epochs, dot, ragged_scan, chunk_parallel_scan]

    def run_all():
        for op in ops:
            op()

    def clear():
        for t in outs.values():
            t.zero_()

    run_all()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in outs.items()}
    for k, t in ref.items():
        assert not torch.isnan(t.float()).any(), f"eager {k} has NaN"
        assert torch.count_nonzero(t) > 0, f"eager {k} is all zero"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run_all()
    torch.cuda.synchronize()
    for r in range(3):
        clear()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.equal(t, ref[k]), f"replay {r}: {k} differs from the eager result"
        clear()
        run_all()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.equal(t, ref[k]), f"eager call after replay {r}: {k} differs"
        print(f"replay {r} ok", flush=True)
