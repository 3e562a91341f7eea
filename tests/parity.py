"""Shared helpers of the GPU parity tests: the comparison metric and the
bar it is held to.

Metric (a reading: an element-wise relative error is undefined near zero):
per (b, h) slice, ||X_gpu - X_ref||_inf / ||X_ref||_inf, maximum over
slices.  Bars: 1e-5 for fp32 inputs; 2e-2 for bf16 inputs with fp32
accumulation.
"""
import numpy as np
import pytest
import torch

TOL = {"f32": 1e-5, "bf16": 2e-2}


def gpu_available() -> bool:
    return torch.cuda.is_available()


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")


def slice_rel_err(got, ref) -> float:
    """max over leading (b,h) slices of ||got-ref||_inf / ||ref||_inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.ndim <= 2:
        got, ref = got[None], ref[None]
    lead = int(np.prod(got.shape[:2])) if got.ndim >= 3 else 1
    g = got.reshape(lead, -1)
    r = ref.reshape(lead, -1)
    num = np.max(np.abs(g - r), axis=1)
    den = np.maximum(np.max(np.abs(r), axis=1), 1e-300)
    return float(np.max(num / den))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def dtype_key(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def banner(msg: str) -> None:
    # names the case before each GPU step, flushed, so a run that dies
    # still says what it was doing
    print(f"[gpu-case] {msg}", flush=True)
