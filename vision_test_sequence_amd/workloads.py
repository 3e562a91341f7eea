"""Seeded synthetic inputs for the TTT layer, shared by the tests, the smoke
check and the benchmark.

This module only draws random numbers and casts them; it holds none of the
layer's arithmetic.  Both the HIP path and the fp64 oracle consume the exact
tensors it returns (the oracle widens the cast values to float64).

Recipe (stated once, used everywhere):
  * generator ``numpy.random.default_rng(seed)`` (PCG64), all draws in fp64;
  * draw order: K, Q, V as [B,H,N,d]; W0 [H,d,d]; w0 [H,d,3,3]; eta [H];
    dZ [B,H,N,d] (only when the workload has a backward);
  * K, Q ~ N(0, 1/d) or, for the high-resolution workloads, N(0,1) rows
    scaled to unit L2 norm per token; V ~ N(0,1); W0 ~ N(0, 1/d);
    w0 ~ N(0, 1/9); eta fixed at 1.0 or ~ U[0.5, 2] per head; dZ ~ N(0,1);
  * cast to float32, then (bf16 workloads) to bfloat16 with round-to-nearest-
    even.  W0, w0 and eta stay float32;
  * two-layer MLP inner model (``draw_mlp_weights``), its own generator
    ``default_rng(seed)``: W1 [H, hidden, d] ~ N(0, 1/d), then W2
    [H, d, hidden] ~ N(0, 1/hidden), float32.

The workloads stand in for the pages' resolutions (224x224 -> 14x14 tokens,
1248x1248 -> 78x78, 1280x1280 -> 80x80, ViT-B at 1024x1024 -> 64x64) with
ViT-T/S/B head shapes (model dim = heads x 64).  No dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

LINEAR = "linear"
DWCONV = "dwconv3x3"


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str                  # "f32" or "bf16"
    B: int
    H: int
    grid_h: int
    grid_w: int
    d: int = 64
    heads: tuple = ()           # inner-model kind per head
    unit_rows: bool = False     # K, Q rows L2-normalised per token
    eta_fixed: Optional[float] = 1.0   # None -> U[0.5, 2] per head
    minibatch: int = 0          # > 0: mini-batch bidirectional scan
    backward: bool = False      # draws dZ as well

    @property
    def N(self) -> int:
        return self.grid_h * self.grid_w

    def head_indices(self, kind: str) -> List[int]:
        return [h for h, k in enumerate(self.heads) if k == kind]


WORKLOADS: Dict[str, Workload] = {
    # 224x224 image, 14x14 tokens, fp32: one linear head and one conv head.
    "tiny_f32": Workload("tiny_f32", 0, "f32", 1, 2, 14, 14, heads=(LINEAR, DWCONV)),
    # ViT^3-T shaped batch at 224x224: 128 images, 3 heads of 64.
    "vit3t_224_bf16": Workload("vit3t_224_bf16", 1, "bf16", 128, 3, 14, 14,
                               heads=(LINEAR, LINEAR, DWCONV), eta_fixed=None),
    # 1248x1248 image stack (16x16 patches -> 78x78 = 6084 tokens).
    "vit3t_1248_bf16": Workload("vit3t_1248_bf16", 2, "bf16", 8, 3, 78, 78,
                                heads=(LINEAR, LINEAR, DWCONV), unit_rows=True),
    # Vision-TTT-S shaped bidirectional mini-batch scan at 1280x1280.
    "vittt_s_1280_bf16": Workload("vittt_s_1280_bf16", 3, "bf16", 4, 6, 80, 80,
                                  heads=(LINEAR,) * 6, unit_rows=True, minibatch=16),
    # ViT-B shaped forward + backward at 1024x1024 (64x64 tokens).
    "vitb_1024_fwdbwd_bf16": Workload("vitb_1024_fwdbwd_bf16", 4, "bf16", 16, 12, 64, 64,
                                      heads=(LINEAR,) * 12, eta_fixed=None, backward=True),
}


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return x / np.maximum(n, 1e-30)


def draw(B: int, H: int, N: int, d: int = 64, *, seed: int, dtype: str = "bf16",
         unit_rows: bool = False, eta_fixed: Optional[float] = 1.0,
         backward: bool = False) -> Dict[str, torch.Tensor]:
    """Draw one input set with the recipe in the module docstring.

    Returns CPU tensors: K, Q, V ([B,H,N,d], dtype), W0 [H,d,d], w0 [H,d,3,3],
    eta [H] (float32) and dZ ([B,H,N,d], dtype) when ``backward``.
    """
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    if unit_rows:
        K = _unit_rows(rng.standard_normal(shape))
        Q = _unit_rows(rng.standard_normal(shape))
    else:
        K = rng.standard_normal(shape) / np.sqrt(d)
        Q = rng.standard_normal(shape) / np.sqrt(d)
    V = rng.standard_normal(shape)
    W0 = rng.standard_normal((H, d, d)) / np.sqrt(d)
    w0 = rng.standard_normal((H, d, 3, 3)) / 3.0
    if eta_fixed is None:
        eta = rng.uniform(0.5, 2.0, size=(H,))
    else:
        eta = np.full((H,), float(eta_fixed))
    out = {
        "K": _cast(K, dtype), "Q": _cast(Q, dtype), "V": _cast(V, dtype),
        "W0": _cast(W0, "f32"), "w0": _cast(w0, "f32"), "eta": _cast(eta, "f32"),
    }
    if backward:
        out["dZ"] = _cast(rng.standard_normal(shape), dtype)
    return out


def draw_mlp_weights(H: int, hidden: int, d: int = 64, *, seed: int) -> Dict[str, torch.Tensor]:
    """W1 [H, hidden, d] and W2 [H, d, hidden] of the two-layer MLP inner
    model (float32, CPU), with the recipe in the module docstring."""
    rng = np.random.default_rng(seed)
    W1 = rng.standard_normal((H, hidden, d)) / np.sqrt(d)
    W2 = rng.standard_normal((H, d, hidden)) / np.sqrt(hidden)
    return {"W1": _cast(W1, "f32"), "W2": _cast(W2, "f32")}


def make(name: str, seed_offset: int = 0, **overrides) -> Dict[str, torch.Tensor]:
    """Inputs of a named workload (optionally with a different seed or shape)."""
    w = WORKLOADS[name]
    B = overrides.get("B", w.B)
    H = overrides.get("H", w.H)
    return draw(B, H, w.N, w.d, seed=w.seed + seed_offset, dtype=w.dtype,
                unit_rows=w.unit_rows, eta_fixed=w.eta_fixed, backward=w.backward)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a (possibly bf16) tensor to a float64 array."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)
