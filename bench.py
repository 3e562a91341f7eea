#!/usr/bin/env python3
"""Benchmark of the MI355X TTT layer.

One step = one pass of the layer's hot path over one batch of the
1248x1248 image stack (B=8, H=3 heads of d=64, 78x78 = 6084 tokens, bf16):
heads 0-1 take one full-batch step of the linear inner model, head 2 one
full-batch step of the 3x3 depthwise inner model, each followed by its
apply -- one ttt_layer_fullbatch call, which runs them as one kernel
(layer_fused).  The two kernels of the separate calls (ttt_linear_fullbatch,
ttt_dwconv3x3_fullbatch) are timed too.

Inputs are resident in HBM before timing and rotate over 5 independent sets
(> 256 MB together, so the 256 MB Infinity Cache cannot hold them between
uses).  The timed steps are captured in one HIP graph and replayed: one
Python call through the binding takes about as long as the layer kernel, so
eager calls would time the host (their rate is reported alongside).  Prints one JSON line: whole-layer tokens/s, the roofline of the
dominant kernel (the step's one kernel), the other rows of the path on their
own workloads (the mini-batch bidirectional scan at 1280x1280, the forward
and backward of the linear step at ViT-B 1024x1024), and the fp64 oracle
timed on the host.

The headline is the median of REPLAYS replays of one graph of K steps
(p10 and p90 reported beside it); every other row is graph-replayed too,
over rotating input sets where one set would fit the Infinity Cache.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores

WORKLOAD = "vit3t_1248_bf16"
SCAN_WORKLOAD = "vittt_s_1280_bf16"
BWD_WORKLOAD = "vitb_1024_fwdbwd_bf16"
METRIC = "TTT-layer tokens/s at N=6084, H=3, d=64 bf16; % MFMA / HBM roofline"
NSETS = 5
REPLAYS = 7                      # graph replays of the headline (median, p10, p90)
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per launch of the layer kernel from rocprofv3 FETCH_SIZE /
# WRITE_SIZE runs, stored with the hash of the sources they were taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer_fused_vit3t_1248_traffic.md")
KERNEL_SOURCES = ["vision_test_sequence_amd/csrc/linear_fullbatch.hip",
                  "vision_test_sequence_amd/csrc/conv_body.hpp",
                  "vision_test_sequence_amd/csrc/dwconv3x3.hip",
                  "vision_test_sequence_amd/csrc/common.hpp",
                  "vision_test_sequence_amd/csrc/api.cpp"]
COPY_BYTES = 256 << 20           # plain copy kernel run once for the counter scale


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the scan and backward rows")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None if
    the kernel sources changed since the counters were taken."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"source-hash:\s*([0-9a-f]+)", txt)
    t = re.search(r"traffic-bytes-per-launch:\s*([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def layer_algorithmic(w):
    """Bytes and flops one layer step must move / perform (per kernel)."""
    N, d, B = w.N, w.d, w.B
    lin_heads = len(w.head_indices("linear"))
    conv_heads = len(w.head_indices("dwconv3x3"))
    esz = 2
    lin_bytes = 4 * B * lin_heads * N * d * esz          # read K, V, Q; write Z
    conv_bytes = 4 * B * conv_heads * N * d * esz
    lin_flops = B * lin_heads * (6 * N * d * d + 2 * d ** 3)  # Gram 4Nd^2, apply 2Nd^2, W0 A
    conv_flops = B * conv_heads * 55 * N * d
    return lin_bytes, conv_bytes, lin_flops, conv_flops


def time_calls(torch, fn, n):
    """Average wall time of n back-to-back calls on the current stream
    (HIP events around the whole run), in ms."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def time_graphed(torch, fn, n, replays=1):
    """Average time per call of n calls captured in one HIP graph
    (torch.cuda.graph), in ms, for each of `replays` timed replays (a list),
    between HIP events on the replay stream.  The layer's kernels take
    about as long as one Python call through the binding, so eager
    back-to-back calls would measure the host; the graph launches the same
    kernels with the same arguments without it.  A warm-up on a side stream
    precedes the capture, as torch asks; an untimed replay precedes the
    timed ones."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(n, 2 * NSETS)):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    # captured on the warm-up stream: the binding's workspace for that
    # stream exists already, so nothing is allocated inside the capture
    with torch.cuda.graph(graph, stream=side):
        for i in range(n):
            fn(i)
    graph.replay()  # untimed
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n)
    del graph
    return times if replays > 1 else times[0]


def spread(times):
    """median, p10, p90 of a list of per-call times (ms)."""
    import numpy as np
    t = np.asarray(times, dtype=np.float64)
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def _row(us, nbytes, tokens, extra=None):
    r = {"us_per_call": us, "tokens_per_s": tokens / (us * 1e-6), "algorithmic_bytes": nbytes,
         "gbs": nbytes / (us * 1e-6) / 1e9, "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    r.update(extra or {})
    return r


def rows(torch, vt, wl, dev, n=40):
    """The other rows of the path on their own workloads, each graph-
    replayed (n calls per graph, median of 3 replays) over input sets that
    rotate where one set would fit the Infinity Cache."""
    out = {}
    med = lambda f, k=n: spread(time_graphed(torch, f, k, replays=3))[0]
    # mini-batch bidirectional scan, 1280x1280, b = 16 (and b = 64)
    w = wl.WORKLOADS[SCAN_WORKLOAD]
    sets = []
    for sidx in range(4):  # 4 x 78.6 MB > the 256 MB Infinity Cache
        inp = wl.make(SCAN_WORKLOAD, seed_offset=1000 * sidx)
        g = {k: inp[k].to(dev) for k in ("K", "Q", "V", "W0", "eta")}
        g["Z"] = torch.empty_like(g["Q"])
        sets.append(g)
    nbytes = 4 * w.B * w.H * w.N * w.d * 2
    for b in (w.minibatch, 64):
        f = lambda i, b=b: vt.ttt_linear_minibatch_bidir(sets[i % 4]["K"], sets[i % 4]["Q"], sets[i % 4]["V"],
                                                         sets[i % 4]["W0"], sets[i % 4]["eta"], b, 0,
                                                         Z=sets[i % 4]["Z"])
        ms = med(f)
        flops = w.B * w.H * w.N * 2 * (6 * w.d ** 2 + 4 * min(b, 16) * w.d)
        out[f"scan_bidir_b{b}"] = _row(ms * 1e3, nbytes, w.B * w.N, {
            "workload": f"{SCAN_WORKLOAD}: B={w.B}, H={w.H}, {w.grid_h}x{w.grid_w} N={w.N}, b={b}, "
                        "both directions averaged, 4 input sets rotated",
            "tflops": flops / (ms * 1e-3) / 1e12})
    del sets
    # one image of the same workload: few chains, so the scan is cut into
    # segments (chunk-parallel); also timed as one walk per chain
    one = []
    for sidx in range(4):
        inp = wl.draw(1, w.H, w.N, seed=w.seed + 1000 * sidx, dtype="bf16", unit_rows=True)
        g = {k: inp[k].to(dev) for k in ("K", "Q", "V", "W0", "eta")}
        g["Z"] = torch.empty_like(g["Q"])
        one.append(g)
    f = lambda i: vt.ttt_linear_minibatch_bidir(one[i % 4]["K"], one[i % 4]["Q"], one[i % 4]["V"], one[i % 4]["W0"],
                                                one[i % 4]["eta"], w.minibatch, 0, Z=one[i % 4]["Z"])
    ms = med(f)
    prev = os.environ.get("TTT_SCAN_SEGMENTS")
    os.environ["TTT_SCAN_SEGMENTS"] = "1"
    try:
        ms1 = med(f)
    finally:
        if prev is None:
            os.environ.pop("TTT_SCAN_SEGMENTS", None)
        else:
            os.environ["TTT_SCAN_SEGMENTS"] = prev
    out["scan_bidir_b16_one_image"] = _row(ms * 1e3, 4 * w.H * w.N * w.d * 2, w.N, {
        "workload": f"{SCAN_WORKLOAD} one image: B=1, H={w.H}, N={w.N}, b={w.minibatch}, both directions, "
                    "chunk-parallel (segments planned per chain)",
        "one_walk_us": ms1 * 1e3})
    del one
    # forward (saving A, G) and backward of the linear step, ViT-B 1024x1024
    w = wl.WORKLOADS[BWD_WORKLOAD]
    inp = wl.make(BWD_WORKLOAD)
    K, Q, V, dZ = (inp[k].to(dev) for k in ("K", "Q", "V", "dZ"))
    W0, eta = inp["W0"].to(dev), inp["eta"].to(dev)
    B, H, N, d = K.shape
    saved = torch.empty((B, H, 2, d, d), dtype=torch.float32, device=dev)
    Z = torch.empty_like(Q)
    outs = [torch.empty_like(K) for _ in range(3)]
    dW0 = torch.empty((H, d, d), dtype=torch.float32, device=dev)
    deta = torch.empty((H,), dtype=torch.float32, device=dev)
    fw = lambda i: vt.ttt_linear_fullbatch(K, Q, V, W0, eta, Z=Z, saved=saved)
    bw = lambda i: vt.ttt_linear_fullbatch_bwd(K, Q, V, W0, eta, dZ, saved=saved, dK=outs[0],
                                               dQ=outs[1], dV=outs[2], dW0=dW0, deta=deta)
    ms_f = med(fw, 10)  # (one set: 1.1 GB per forward + backward, beyond the Infinity Cache)
    ms_b = med(bw, 10)
    fb = 4 * B * H * N * d * 2
    bb = 7 * B * H * N * d * 2
    out["fwd_bwd"] = {
        "workload": f"{BWD_WORKLOAD}: B={B}, H={H}, {w.grid_h}x{w.grid_w} N={N}, forward saves "
                    "A and G, backward returns dK, dQ, dV, dW0, deta",
        "fwd_us": ms_f * 1e3, "bwd_us": ms_b * 1e3,
        "fwd_gbs": fb / (ms_f * 1e-3) / 1e9, "bwd_gbs": bb / (ms_b * 1e-3) / 1e9,
        "hbm_frac": (fb + bb) / ((ms_f + ms_b) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "bwd_hbm_frac": bb / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "tokens_per_s": B * N / ((ms_f + ms_b) * 1e-3),
    }
    del K, Q, V, dZ, Z, outs, saved
    # the 1248x1248 layer's other operations: conv-head backward, the
    # gradient magnitude map of the linear heads, dot-product loss and two
    # full-batch steps of the linear heads
    w = wl.WORKLOADS[WORKLOAD]
    lin = w.head_indices("linear")
    l0, l1, c = lin[0], lin[-1] + 1, w.head_indices("dwconv3x3")[0]
    gs = []
    for sidx in range(NSETS):
        inp = wl.draw(w.B, w.H, w.N, seed=w.seed + 1000 * sidx, dtype="bf16", unit_rows=True, backward=True)
        g = {k: v.to(dev) for k, v in inp.items()}
        g["out"] = [torch.empty_like(g["K"][:, c:c + 1]) for _ in range(3)]
        g["Z"] = torch.empty_like(g["Q"])
        g["gmm"] = torch.empty((w.B, l1 - l0, w.N), dtype=torch.float32, device=dev)
        g["W0l"], g["etal"] = g["W0"][l0:l1].contiguous(), g["eta"][l0:l1].contiguous()
        g["w0c"], g["etac"] = g["w0"][c:c + 1].contiguous(), g["eta"][c:c + 1].contiguous()
        gs.append(g)
    conv_dw0 = torch.empty((1, 64, 3, 3), dtype=torch.float32, device=dev)
    conv_deta = torch.empty((1,), dtype=torch.float32, device=dev)
    cb = lambda i: vt.ttt_dwconv3x3_fullbatch_bwd(
        gs[i % NSETS]["K"][:, c:c + 1], gs[i % NSETS]["Q"][:, c:c + 1], gs[i % NSETS]["V"][:, c:c + 1],
        gs[i % NSETS]["w0c"], gs[i % NSETS]["etac"], gs[i % NSETS]["dZ"][:, c:c + 1], w.grid_h, w.grid_w,
        dK=gs[i % NSETS]["out"][0], dQ=gs[i % NSETS]["out"][1], dV=gs[i % NSETS]["out"][2], dw0=conv_dw0,
        deta=conv_deta)
    ms = med(cb)
    out["dwconv_bwd"] = _row(ms * 1e3, 7 * w.B * w.N * w.d * 2, w.B * w.N, {
        "workload": f"{WORKLOAD} conv head: B={w.B}, {w.grid_h}x{w.grid_w}, g recomputed, "
                    f"{NSETS} input sets rotated"})
    lv = lambda g: (g["K"][:, l0:l1], g["Q"][:, l0:l1], g["V"][:, l0:l1], g["W0l"], g["etal"])
    gm = lambda i: vt.ttt_linear_gradient_magnitude(gs[i % NSETS]["K"][:, l0:l1], gs[i % NSETS]["V"][:, l0:l1],
                                                    gs[i % NSETS]["W0l"], out=gs[i % NSETS]["gmm"])
    ms = med(gm)
    out["gradient_magnitude_map"] = _row(ms * 1e3, w.B * (l1 - l0) * w.N * (2 * w.d * 2 + 4), w.B * w.N, {
        "workload": f"{WORKLOAD} linear heads: K, V read, one fp32 norm written per token and head"})
    dl = lambda i: vt.ttt_linear_fullbatch(*lv(gs[i % NSETS]), Z=gs[i % NSETS]["Z"][:, l0:l1], loss=vt.LOSS_DOT)
    ms = med(dl)
    out["linear_dot_loss"] = _row(ms * 1e3, 4 * w.B * (l1 - l0) * w.N * w.d * 2, w.B * w.N, {
        "workload": f"{WORKLOAD} linear heads, dot-product loss (one launch, G exchange)"})
    e2 = lambda i: vt.ttt_linear_fullbatch(*lv(gs[i % NSETS]), Z=gs[i % NSETS]["Z"][:, l0:l1], steps=2)
    ms = med(e2)
    out["linear_two_steps"] = _row(ms * 1e3, 4 * w.B * (l1 - l0) * w.N * w.d * 2, w.B * w.N, {
        "workload": f"{WORKLOAD} linear heads, two full-batch steps (one launch: a second G exchange round)"})
    os.environ["TTT_SPLIT_STEPS"] = "1"
    try:
        out["linear_two_steps"]["three_launch_us"] = med(e2) * 1e3
    finally:
        del os.environ["TTT_SPLIT_STEPS"]
    # two-layer SiLU MLP inner model on every head of the stack, widths d and 4d
    for hid in (64, 256):
        mw = {k: v.to(dev) for k, v in wl.draw_mlp_weights(w.H, hid, seed=w.seed + 1).items()}
        ml = lambda i: vt.ttt_mlp_fullbatch(gs[i % NSETS]["K"], gs[i % NSETS]["Q"], gs[i % NSETS]["V"], mw["W1"],
                                            mw["W2"], gs[i % NSETS]["eta"], Z=gs[i % NSETS]["Z"])
        ms = med(ml)
        flops = w.B * w.H * w.N * 14 * w.d * hid
        out[f"mlp_hidden{hid}"] = _row(ms * 1e3, 4 * w.B * w.H * w.N * w.d * 2, w.B * w.N, {
            "workload": f"{WORKLOAD}: B={w.B}, all {w.H} heads a two-layer SiLU MLP of hidden width {hid}, "
                        "one full-batch step then apply",
            "tflops": flops / (ms * 1e-3) / 1e12, "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS})
    del gs
    # backward of the bidirectional scan, 1280x1280, b = 16
    w = wl.WORKLOADS[SCAN_WORKLOAD]
    inp = wl.draw(w.B, w.H, w.N, seed=w.seed, dtype="bf16", unit_rows=True, backward=True)
    g = {k: v.to(dev) for k, v in inp.items()}
    outs = [torch.empty_like(g["K"]) for _ in range(3)]
    dW0 = torch.empty_like(g["W0"])
    deta = torch.empty_like(g["eta"])
    sb = lambda i: vt.ttt_linear_minibatch_bidir_bwd(g["K"], g["Q"], g["V"], g["W0"], g["eta"], g["dZ"],
                                                     w.minibatch, 0, dK=outs[0], dQ=outs[1], dV=outs[2],
                                                     dW0=dW0, deta=deta)
    ms = med(sb, 3)
    out["scan_bidir_bwd_b16"] = _row(ms * 1e3, 7 * w.B * w.H * w.N * w.d * 2, w.B * w.N, {
        "workload": f"{SCAN_WORKLOAD}: B={w.B}, H={w.H}, N={w.N}, b={w.minibatch}, both directions, "
                    "states recomputed"})
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import vision_test_sequence_amd as vt
    from vision_test_sequence_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    vt.lib()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[WORKLOAD]
    lin = w.head_indices("linear")
    cnv = w.head_indices("dwconv3x3")
    l0, l1, c0, c1 = lin[0], lin[-1] + 1, cnv[0], cnv[-1] + 1

    sets = []
    for s in range(NSETS):
        inp = wl.make(WORKLOAD, seed_offset=1000 * s)
        g = {k: v.to(dev) for k, v in inp.items()}
        g["Z"] = torch.empty_like(g["Q"])
        g["W0l"] = g["W0"][l0:l1].contiguous()
        g["etal"] = g["eta"][l0:l1].contiguous()
        g["w0c"] = g["w0"][c0:c1].contiguous()
        g["etac"] = g["eta"][c0:c1].contiguous()
        sets.append((inp, g))
    torch.cuda.synchronize()

    def linear(g):
        vt.ttt_linear_fullbatch(g["K"][:, l0:l1], g["Q"][:, l0:l1], g["V"][:, l0:l1],
                                g["W0l"], g["etal"], Z=g["Z"][:, l0:l1])

    def conv(g):
        vt.ttt_dwconv3x3_fullbatch(g["K"][:, c0:c1], g["Q"][:, c0:c1], g["V"][:, c0:c1],
                                   g["w0c"], g["etac"], w.grid_h, w.grid_w, Z=g["Z"][:, c0:c1])

    def step(g):
        vt.ttt_layer_fullbatch(g["K"][:, l0:l1], g["Q"][:, l0:l1], g["V"][:, l0:l1], g["W0l"], g["etal"],
                               g["K"][:, c0:c1], g["Q"][:, c0:c1], g["V"][:, c0:c1], g["w0c"], g["etac"],
                               w.grid_h, w.grid_w, Zl=g["Z"][:, l0:l1], Zc=g["Z"][:, c0:c1])

    def separate(g):
        linear(g)
        conv(g)

    for i in range(args.warmup):
        step(sets[i % NSETS][1])
    torch.cuda.synchronize()

    # timed region: K layer steps rotating over the input sets, captured in
    # one graph and replayed between HIP events on the replay stream; a step
    # is one launch, so this is also the layer kernel's average launch
    # duration
    step_times = time_graphed(torch, lambda i: step(sets[i % NSETS][1]), args.steps, replays=REPLAYS)
    ms_step, p10_step, p90_step = spread(step_times)
    # the same steps as eager calls from Python (host-bound: reported only)
    eager_ms_step = time_calls(torch, lambda i: step(sets[i % NSETS][1]), args.steps)
    # the two kernels of the separate calls, the same way (average launch
    # duration)
    nk = max(args.steps, 200)
    lin_ms = time_graphed(torch, lambda i: linear(sets[i % NSETS][1]), nk)
    conv_ms = time_graphed(torch, lambda i: conv(sets[i % NSETS][1]), nk)
    sep_ms = time_graphed(torch, lambda i: separate(sets[i % NSETS][1]), nk)
    # warm reference: the same buffers every step (Infinity-Cache resident)
    warm_ms_step = time_graphed(torch, lambda i: step(sets[0][1]), args.steps)

    # one plain device copy of known size: the scale for the HBM byte
    # counters of the profiled runs
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    tokens = w.B * w.N
    lin_bytes, conv_bytes, lin_flops, conv_flops = layer_algorithmic(w)
    achieved = (lin_bytes + conv_bytes) / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{WORKLOAD}: B={w.B} images, H={w.H} heads (0-1 linear full-batch, "
                        f"2 dwconv3x3 full-batch, one ttt_layer_fullbatch call), "
                        f"{w.grid_h}x{w.grid_w} grid N={w.N}, d={w.d}",
            "global_batch": w.B,
            "seq_len": w.N,
            "input_sets_rotated": NSETS,
        },
        "roofline": {
            "kernel": "layer_fused (ttt_layer_fullbatch: heads 0-1 linear, head 2 dwconv3x3, B=8, N=6084)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "algorithmic_bytes": lin_bytes + conv_bytes,
            "avg_launch_us": ms_step * 1e3,
        },
        "timing": {
            "replays": REPLAYS, "steps_per_replay": args.steps,
            "median_us": ms_step * 1e3, "p10_us": p10_step * 1e3, "p90_us": p90_step * 1e3,
        },
        "kernels": {
            "eager_python_us_per_step": eager_ms_step * 1e3,
            "separate_calls_us_per_step": sep_ms * 1e3,
            "linear_us": lin_ms * 1e3,
            "linear_gbs": lin_bytes / (lin_ms * 1e-3) / 1e9,
            "linear_hbm_frac": lin_bytes / (lin_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "linear_tflops": lin_flops / (lin_ms * 1e-3) / 1e12,
            "linear_mfma_frac": lin_flops / (lin_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "dwconv_us": conv_ms * 1e3,
            "dwconv_gbs": conv_bytes / (conv_ms * 1e-3) / 1e9,
            "dwconv_hbm_frac": conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "warm_ms_per_step": warm_ms_step,
        },
    }
    if not args.no_rows:
        out["rows"] = rows(torch, vt, wl, dev)

    # CPU baseline: the fp64 oracle, as it stands, on input set 0 of the
    # same workload, repeated until a few seconds have accumulated; its
    # result also checks the GPU output of that set.
    if not args.no_cpu_baseline:
        import oracle
        inp0, g0 = sets[0]
        step(g0)
        torch.cuda.synchronize()
        Zgpu = wl.to_f64(g0["Z"])
        K, Q, V = (wl.to_f64(inp0[k]) for k in "KQV")
        W0, w0, eta = (wl.to_f64(inp0[k]) for k in ("W0", "w0", "eta"))
        reps, t0 = 0, time.perf_counter()
        while True:
            Zl, _ = oracle.linear_fullbatch(K[:, l0:l1], Q[:, l0:l1], V[:, l0:l1], W0[l0:l1],
                                            eta[l0:l1])
            Zc, _ = oracle.dwconv3x3_fullbatch(K[:, c0:c1], Q[:, c0:c1], V[:, c0:c1], w0[c0:c1],
                                               eta[c0:c1], w.grid_h, w.grid_w)
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= 10.0:
                break
        cores = oracle.max_threads()  # (read before the one-thread run changes it)
        # one thread, on image 0 of the same set (all three heads)
        reps1, t1 = 0, time.perf_counter()
        while True:
            oracle.linear_fullbatch(K[:1, l0:l1], Q[:1, l0:l1], V[:1, l0:l1], W0[l0:l1], eta[l0:l1], threads=1)
            oracle.dwconv3x3_fullbatch(K[:1, c0:c1], Q[:1, c0:c1], V[:1, c0:c1], w0[c0:c1], eta[c0:c1],
                                       w.grid_h, w.grid_w, threads=1)
            reps1 += 1
            el1 = time.perf_counter() - t1
            if el1 >= 5.0:
                break
        out["cpu_baseline"] = {
            "value": tokens * reps / elapsed,
            "unit": "tokens/s",
            "cores": cores,
            "kind": "oracle",
            "sample": f"the whole workload (input set 0: {w.B} images x {w.H} heads x {w.N} "
                      f"tokens), {reps} repetitions in {elapsed:.2f} s; fp64 C loops, "
                      "OpenMP over (image, head) slices",
            "one_thread": {"value": w.N * reps1 / el1, "unit": "tokens/s",
                           "sample": f"image 0 of input set 0 (3 heads x {w.N} tokens), {reps1} "
                                     f"repetitions in {el1:.2f} s on one thread"},
        }

        def rel(got, ref):  # per-slice inf-norm relative error, max over slices
            g = got.reshape(got.shape[0] * got.shape[1], -1)
            r = ref.reshape(ref.shape[0] * ref.shape[1], -1)
            return float(np.max(np.max(np.abs(g - r), 1) / np.maximum(np.max(np.abs(r), 1), 1e-300)))

        out["parity_vs_oracle"] = {
            "linear_heads_max_rel_err": rel(Zgpu[:, l0:l1], Zl),
            "dwconv_head_max_rel_err": rel(Zgpu[:, c0:c1], Zc),
            "tolerance": 2e-2,
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
