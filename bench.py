#!/usr/bin/env python3
"""Benchmark of the MI355X TTT layer.

One step = one pass of the layer's hot path over one batch of the
1248x1248 image stack (B=8, H=3 heads of d=64, 78x78 = 6084 tokens, bf16):
heads 0-1 take one full-batch step of the linear inner model
(ttt_linear_fullbatch), head 2 one full-batch step of the 3x3 depthwise
inner model (ttt_dwconv3x3_fullbatch), each followed by its apply.

Inputs are resident in HBM before timing and rotate over 5 independent sets
(> 256 MB together, so the 256 MB Infinity Cache cannot hold them between
uses).  Prints one JSON line: whole-layer tokens/s plus the roofline of the
dominant kernel (the linear step) and the fp64 oracle timed on the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores

WORKLOAD = "vit3t_1248_bf16"
METRIC = "TTT-layer tokens/s at N=6084, H=3, d=64 bf16; % MFMA / HBM roofline"
NSETS = 5


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def algorithmic(w):
    """Bytes and flops one step must move / perform (per launch kind)."""
    N, d, B = w.N, w.d, w.B
    lin_heads = len(w.head_indices("linear"))
    conv_heads = len(w.head_indices("dwconv3x3"))
    esz = 2
    lin_bytes = 4 * B * lin_heads * N * d * esz          # read K, V, Q; write Z
    conv_bytes = 4 * B * conv_heads * N * d * esz
    lin_flops = B * lin_heads * (6 * N * d * d + 2 * d ** 3)  # Gram 4Nd^2, apply 2Nd^2, W0 A
    conv_flops = B * conv_heads * 55 * N * d
    return lin_bytes, conv_bytes, lin_flops, conv_flops


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
        sets.append((inp, g))
    torch.cuda.synchronize()

    def step(g, ev=None):
        if ev is not None:
            ev[0].record()
        vt.ttt_linear_fullbatch(g["K"][:, l0:l1], g["Q"][:, l0:l1], g["V"][:, l0:l1],
                                g["W0l"], g["etal"], Z=g["Z"][:, l0:l1])
        if ev is not None:
            ev[1].record()
        vt.ttt_dwconv3x3_fullbatch(g["K"][:, c0:c1], g["Q"][:, c0:c1], g["V"][:, c0:c1],
                                   g["w0c"], g["etac"], w.grid_h, w.grid_w, Z=g["Z"][:, c0:c1])
        if ev is not None:
            ev[2].record()

    for _, g in sets:
        g["W0l"] = g["W0"][l0:l1].contiguous()
        g["etal"] = g["eta"][l0:l1].contiguous()
        g["w0c"] = g["w0"][c0:c1].contiguous()
        g["etac"] = g["eta"][c0:c1].contiguous()

    for i in range(args.warmup):
        step(sets[i % NSETS][1])
    torch.cuda.synchronize()

    # timed region: K steps rotating over the input sets; per-launch events
    # on the launch stream (torch's current stream) give each kernel's time
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(sets[i % NSETS][1], evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    lin_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    conv_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    # warm reference: the same buffers every step (Infinity-Cache resident)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(sets[0][1])
    t_end.record()
    torch.cuda.synchronize()
    warm_ms_step = t_start.elapsed_time(t_end) / args.steps

    tokens = w.B * w.N
    lin_bytes, conv_bytes, lin_flops, conv_flops = algorithmic(w)
    achieved = lin_bytes / (lin_ms * 1e-3) / 1e9
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
                        f"2 dwconv3x3 full-batch), {w.grid_h}x{w.grid_w} grid N={w.N}, d={w.d}",
            "global_batch": w.B,
            "seq_len": w.N,
            "input_sets_rotated": NSETS,
        },
        "roofline": {
            "kernel": "lin_fwd_kernel (ttt_linear_fullbatch, heads 0-1)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "algorithmic_bytes": lin_bytes,
            "avg_launch_us": lin_ms * 1e3,
        },
        "kernels": {
            "linear_us": lin_ms * 1e3,
            "linear_tflops": lin_flops / (lin_ms * 1e-3) / 1e12,
            "linear_mfma_frac": lin_flops / (lin_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "dwconv_us": conv_ms * 1e3,
            "dwconv_gbs": conv_bytes / (conv_ms * 1e-3) / 1e9,
            "dwconv_hbm_frac": conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "layer_hbm_frac": (lin_bytes + conv_bytes) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "warm_ms_per_step": warm_ms_step,
        },
    }

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
            if elapsed >= 5.0 or reps >= 30:
                break
        out["cpu_baseline"] = {
            "value": tokens * reps / elapsed,
            "unit": "tokens/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"the whole workload (input set 0: {w.B} images x {w.H} heads x {w.N} "
                      f"tokens), {reps} repetitions in {elapsed:.2f} s; fp64 C loops, "
                      "OpenMP over (image, head) slices",
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
