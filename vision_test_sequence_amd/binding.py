"""ctypes binding of libttt.so (include/ttt.h).

Argument marshalling only: torch tensors are turned into device pointers,
element strides and the current HIP stream; the workspace is a zero-filled
torch byte tensor kept per (device, op).  Every step of the layer runs in
the library's HIP kernels.  A missing library raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libttt.so")

TTT_F32 = 0
TTT_BF16 = 1
BIDIR_AVG = 0
FORWARD_ONLY = 1
BACKWARD_ONLY = 2
OP_LINEAR_FULLBATCH = 0
OP_DWCONV3X3_FULLBATCH = 1
OP_LINEAR_MINIBATCH_BIDIR = 2
OP_LINEAR_FULLBATCH_BWD = 3
OP_LAYER_FULLBATCH = 4
OP_DWCONV3X3_FULLBATCH_BWD = 5
OP_LINEAR_MINIBATCH_BIDIR_BWD = 6
OP_MLP_FULLBATCH = 7

KERNEL_LIN_RESIDENT = 1
KERNEL_LIN_RESIDENT_GX = 2
KERNEL_LIN_STREAM = 3
KERNEL_DWCONV = 4

STATUS_NAMES = [
    "TTT_OK", "TTT_ERR_NULL_POINTER", "TTT_ERR_BAD_SHAPE", "TTT_ERR_BAD_STRIDE",
    "TTT_ERR_MISALIGNED", "TTT_ERR_UNSUPPORTED", "TTT_ERR_ALIASING",
    "TTT_ERR_WORKSPACE_TOO_SMALL", "TTT_ERR_HIP",
]

EXPORTED = ("ttt_workspace_size", "ttt_status_string", "ttt_layer_workspace_size", "ttt_linear_fullbatch",
            "ttt_dwconv3x3_fullbatch", "ttt_linear_minibatch_bidir", "ttt_linear_fullbatch_bwd",
            "ttt_layer_fullbatch", "ttt_plan_query", "ttt_layer_plan_query",
            "ttt_workspace_exchange_failed", "ttt_workspace_reset", "ttt_linear_fullbatch_noalloc", "ttt_dwconv3x3_fullbatch_bwd",
            "ttt_linear_gradient_magnitude", "ttt_linear_minibatch_bidir_bwd", "ttt_mlp_fullbatch")


class TTTError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name}")
        self.name = name


class View(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


LOSS_L2 = 0
LOSS_DOT = 1


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("minibatch", ctypes.c_int32), ("mode", ctypes.c_int),
                ("loss", ctypes.c_int), ("steps", ctypes.c_int32), ("w0_per_direction", ctypes.c_int32),
                ("hidden", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("splits", ctypes.c_int32), ("xcd_local", ctypes.c_int32),
                ("fused", ctypes.c_int32)]


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libttt.so with argument types declared (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build it with `python -m vision_test_sequence_amd.build`"
                    " (there is no CPU fallback)")
            L = ctypes.CDLL(_LIB_PATH)
            vp, sz, fp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
            P = ctypes.POINTER(Problem)
            L.ttt_workspace_size.argtypes = [ctypes.c_int, P]
            L.ttt_workspace_size.restype = sz
            L.ttt_status_string.argtypes = [ctypes.c_int]
            L.ttt_status_string.restype = ctypes.c_char_p
            L.ttt_layer_workspace_size.argtypes = [P, P]
            L.ttt_layer_workspace_size.restype = sz
            L.ttt_linear_fullbatch.argtypes = [P, View, View, View, fp, fp, View, fp, vp, sz, vp]
            L.ttt_dwconv3x3_fullbatch.argtypes = [P, View, View, View, fp, fp, View, fp, vp, sz, vp]
            L.ttt_linear_minibatch_bidir.argtypes = [P, View, View, View, fp, fp, View, vp, sz, vp]
            L.ttt_linear_fullbatch_bwd.argtypes = [P, View, View, View, fp, fp, View, fp, View, View,
                                                   View, fp, fp, vp, sz, vp]
            L.ttt_layer_fullbatch.argtypes = [P, View, View, View, fp, fp, View, P, View, View, View, fp, fp,
                                              View, vp, sz, vp]
            L.ttt_plan_query.argtypes = [ctypes.c_int, P, ctypes.c_int, ctypes.POINTER(PlanInfo)]
            L.ttt_layer_plan_query.argtypes = [P, P, ctypes.POINTER(ctypes.c_int32)]
            L.ttt_workspace_exchange_failed.argtypes = [ctypes.c_int, vp, sz, ctypes.POINTER(ctypes.c_int32), vp]
            L.ttt_workspace_reset.argtypes = [vp, sz, vp]
            L.ttt_linear_fullbatch_noalloc.argtypes = [P, View, View, View, fp, fp, View, fp, vp]
            L.ttt_dwconv3x3_fullbatch_bwd.argtypes = [P, View, View, View, fp, fp, View, fp, View, View,
                                                      View, fp, fp, vp, sz, vp]
            L.ttt_linear_gradient_magnitude.argtypes = [P, View, View, fp, fp, vp]
            L.ttt_linear_minibatch_bidir_bwd.argtypes = [P, View, View, View, fp, fp, View, View, View, View,
                                                         fp, fp, vp, sz, vp]
            L.ttt_mlp_fullbatch.argtypes = [P, View, View, View, fp, fp, fp, View, vp, sz, vp]
            for f in EXPORTED[3:]:
                getattr(L, f).restype = ctypes.c_int
            _lib = L
    return _lib


# ------------------------------------------------------------ marshalling --
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TTT_F32
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def view(t: torch.Tensor) -> View:
    s = t.stride()
    if len(s) != 4:
        raise ValueError("views are [B,H,N,d] tensors")
    if s[3] != 1 and t.shape[3] > 1:
        raise ValueError("the d channels of a view must be contiguous")
    return View(t.data_ptr(), s[0], s[1], s[2])


def problem(K: torch.Tensor, grid: Tuple[int, int] = (0, 0), minibatch: int = 0,
            mode: int = BIDIR_AVG, loss: int = LOSS_L2, steps: int = 1, w0_per_direction: int = 0,
            hidden: int = 0) -> Problem:
    B, H, N, d = K.shape
    return Problem(B, H, N, d, _dtype_code(K), grid[0], grid[1], minibatch, mode, loss, steps,
                   w0_per_direction, hidden)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_ws: Dict[Tuple[int, int, int], torch.Tensor] = {}


def workspace(op: int, prob: Optional[Problem], device: torch.device, need: Optional[int] = None
              ) -> Tuple[Optional[int], int]:
    """Zero-filled scratch for `op`, cached per (device, stream, op); grows on
    demand.  The library leaves its counters at zero after every call, so one
    buffer serves consecutive calls of that op on one stream (calls on
    different streams get different buffers: they may overlap in time)."""
    if need is None:
        need = int(lib().ttt_workspace_size(op, ctypes.byref(prob)))
    if need == 0:
        return None, 0
    dev = device.index if device.index is not None else torch.cuda.current_device()
    key = (dev, _stream(torch.device("cuda", dev)), op)
    buf = _ws.get(key)
    if buf is None or buf.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            # the zero-fill would be recorded into the graph
            raise RuntimeError("no workspace for this stream yet: run the call once on the capture "
                               "stream before capturing it (torch.cuda.graph(..., stream=s))")
        buf = torch.zeros(need, dtype=torch.uint8, device=device)
        _ws[key] = buf
    return buf.data_ptr(), buf.numel()


def exchange_failures():
    """(device, stream, op) of every cached workspace whose split-slice
    exchange has failed (its slices' outputs are NaN until reset); waits for
    each workspace's stream."""
    bad = []
    for (dev, stream, op), buf in list(_ws.items()):
        failed = ctypes.c_int32(0)
        with torch.cuda.device(dev):
            st = lib().ttt_workspace_exchange_failed(op, buf.data_ptr(), buf.numel(), ctypes.byref(failed), stream)
        _check(st, "ttt_workspace_exchange_failed")
        if failed.value:
            bad.append((dev, stream, op))
    return bad


def reset_workspaces() -> None:
    """Zero-fill every cached workspace on its stream (clears failed exchanges)."""
    for (dev, stream, op), buf in list(_ws.items()):
        with torch.cuda.device(dev):
            _check(lib().ttt_workspace_reset(buf.data_ptr(), buf.numel(), stream), "ttt_workspace_reset")


def plan_linear(B: int, H: int, N: int, dtype: int = TTT_BF16, with_saved: bool = False,
                steps: int = 1) -> PlanInfo:
    """Kernel, splits per slice and exchange protocol of ttt_linear_fullbatch
    for this shape on the current device (with steps > 1, `fused` says
    whether the steps run inside one launch)."""
    p = Problem(B, H, N, 64, dtype, 0, 0, 0, 0, LOSS_L2, steps, 0, 0)
    out = PlanInfo()
    _check(lib().ttt_plan_query(OP_LINEAR_FULLBATCH, ctypes.byref(p), int(with_saved), ctypes.byref(out)),
           "ttt_plan_query")
    return out


def plan_dwconv(B: int, H: int, grid_h: int, grid_w: int, dtype: int = TTT_BF16) -> PlanInfo:
    p = Problem(B, H, grid_h * grid_w, 64, dtype, grid_h, grid_w, 0, 0)
    out = PlanInfo()
    _check(lib().ttt_plan_query(OP_DWCONV3X3_FULLBATCH, ctypes.byref(p), 0, ctypes.byref(out)),
           "ttt_plan_query")
    return out


def plan_layer_fused(lin: Tuple[int, int, int], conv: Tuple[int, int, int, int], dtype: int = TTT_BF16) -> bool:
    """Whether ttt_layer_fullbatch runs as one launch: lin = (B, H, N),
    conv = (B, H, grid_h, grid_w)."""
    pl = Problem(lin[0], lin[1], lin[2], 64, dtype, 0, 0, 0, 0)
    pc = Problem(conv[0], conv[1], conv[2] * conv[3], 64, dtype, conv[2], conv[3], 0, 0)
    f = ctypes.c_int32(0)
    _check(lib().ttt_layer_plan_query(ctypes.byref(pl), ctypes.byref(pc), ctypes.byref(f)),
           "ttt_layer_plan_query")
    return bool(f.value)


def _check(st: int, where: str) -> None:
    if st != 0:
        raise TTTError(st, where)


def _param(t: torch.Tensor, shape, name: str) -> torch.Tensor:
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")
    return t


# ------------------------------------------------------------ entry points --
def ttt_linear_fullbatch(K, Q, V, W0, eta, *, Z=None, saved=None, loss: int = LOSS_L2, steps: int = 1):
    """Full-batch gradient step(s) of the linear inner model, then Z = W q per token.

    K, Q, V: [B,H,N,64] float32/bfloat16 on the GPU; W0 [H,64,64] and eta [H]
    float32.  Z (optional) receives the output; saved (optional, float32
    [B,H,2,64,64]) receives A then G per slice.  loss: LOSS_L2 or LOSS_DOT;
    steps: full-batch steps (saved must be None above one).  Returns Z.
    """
    B, H, N, d = K.shape
    _param(W0, (H, d, d), "W0")
    _param(eta, (H,), "eta")
    if Z is None:
        Z = torch.empty((B, H, N, d), dtype=K.dtype, device=K.device)
    p = problem(K, loss=loss, steps=steps)
    ws, wsb = workspace(OP_LINEAR_FULLBATCH, p, K.device)
    st = lib().ttt_linear_fullbatch(ctypes.byref(p), view(K), view(Q), view(V), W0.data_ptr(),
                                    eta.data_ptr(), view(Z), _ptr(saved), ws, wsb,
                                    _stream(K.device))
    _check(st, "ttt_linear_fullbatch")
    return Z


def ttt_linear_fullbatch_noalloc(K, Q, V, W0, eta, *, Z=None, saved=None):
    """ttt_linear_fullbatch on the library's fixed device scratch (no caller
    workspace).  Calls on one device must not overlap in time.  Returns Z."""
    B, H, N, d = K.shape
    _param(W0, (H, d, d), "W0")
    _param(eta, (H,), "eta")
    if Z is None:
        Z = torch.empty((B, H, N, d), dtype=K.dtype, device=K.device)
    p = problem(K)
    st = lib().ttt_linear_fullbatch_noalloc(ctypes.byref(p), view(K), view(Q), view(V), W0.data_ptr(),
                                            eta.data_ptr(), view(Z), _ptr(saved), _stream(K.device))
    _check(st, "ttt_linear_fullbatch_noalloc")
    return Z


def ttt_dwconv3x3_fullbatch(K, Q, V, w0, eta, grid_h: int, grid_w: int, *, Z=None, saved=None,
                            loss: int = LOSS_L2):
    """One full-batch L2 step of the 3x3 depthwise-conv inner model, then apply.

    Tokens form a row-major grid_h x grid_w map.  w0 [H,64,3,3], eta [H]
    float32; saved (optional, float32 [B,H,64,3,3]) receives g.  Returns Z.
    """
    B, H, N, d = K.shape
    _param(w0, (H, d, 3, 3), "w0")
    _param(eta, (H,), "eta")
    if Z is None:
        Z = torch.empty((B, H, N, d), dtype=K.dtype, device=K.device)
    p = problem(K, grid=(grid_h, grid_w), loss=loss)
    ws, wsb = workspace(OP_DWCONV3X3_FULLBATCH, p, K.device)
    st = lib().ttt_dwconv3x3_fullbatch(ctypes.byref(p), view(K), view(Q), view(V), w0.data_ptr(),
                                       eta.data_ptr(), view(Z), _ptr(saved), ws, wsb,
                                       _stream(K.device))
    _check(st, "ttt_dwconv3x3_fullbatch")
    return Z


def ttt_layer_fullbatch(Kl, Ql, Vl, W0, eta_l, Kc, Qc, Vc, w0, eta_c, grid_h: int, grid_w: int, *,
                        Zl=None, Zc=None, loss: int = LOSS_L2):
    """Both full-batch steps of one layer in one call: ttt_linear_fullbatch on
    (Kl, Ql, Vl, W0, eta_l) and ttt_dwconv3x3_fullbatch on (Kc, Qc, Vc, w0,
    eta_c) over a grid_h x grid_w token map, with the same results; one
    launch when they fit.  Views as in the two calls (the linear and conv
    heads may be head ranges of one tensor).  Returns (Zl, Zc).
    """
    Bl, Hl, N, d = Kl.shape
    Bc, Hc = Kc.shape[0], Kc.shape[1]
    _param(W0, (Hl, d, d), "W0")
    _param(eta_l, (Hl,), "eta_l")
    _param(w0, (Hc, d, 3, 3), "w0")
    _param(eta_c, (Hc,), "eta_c")
    if Zl is None:
        Zl = torch.empty((Bl, Hl, N, d), dtype=Kl.dtype, device=Kl.device)
    if Zc is None:
        Zc = torch.empty(tuple(Kc.shape), dtype=Kc.dtype, device=Kc.device)
    pl = problem(Kl, loss=loss)
    pc = problem(Kc, grid=(grid_h, grid_w), loss=loss)
    need = int(lib().ttt_layer_workspace_size(ctypes.byref(pl), ctypes.byref(pc)))
    ws, wsb = workspace(OP_LAYER_FULLBATCH, None, Kl.device, need)
    st = lib().ttt_layer_fullbatch(ctypes.byref(pl), view(Kl), view(Ql), view(Vl), W0.data_ptr(),
                                   eta_l.data_ptr(), view(Zl), ctypes.byref(pc), view(Kc), view(Qc),
                                   view(Vc), w0.data_ptr(), eta_c.data_ptr(), view(Zc), ws, wsb,
                                   _stream(Kl.device))
    _check(st, "ttt_layer_fullbatch")
    return Zl, Zc


def ttt_linear_minibatch_bidir(K, Q, V, W0, eta, minibatch: int, mode: int = BIDIR_AVG, *, Z=None):
    """Causal mini-batch scans (forward, reverse or their average). Returns Z.

    W0: [H,64,64] shared by both directions, or [2,H,64,64] with the
    forward scan starting from W0[0] and the reversed one from W0[1]."""
    B, H, N, d = K.shape
    w0dir = 1 if W0.dim() == 4 else 0
    _param(W0, (2, H, d, d) if w0dir else (H, d, d), "W0")
    _param(eta, (H,), "eta")
    if Z is None:
        Z = torch.empty((B, H, N, d), dtype=K.dtype, device=K.device)
    p = problem(K, minibatch=minibatch, mode=mode, w0_per_direction=w0dir)
    ws, wsb = workspace(OP_LINEAR_MINIBATCH_BIDIR, p, K.device)
    st = lib().ttt_linear_minibatch_bidir(ctypes.byref(p), view(K), view(Q), view(V),
                                          W0.data_ptr(), eta.data_ptr(), view(Z), ws, wsb,
                                          _stream(K.device))
    _check(st, "ttt_linear_minibatch_bidir")
    return Z


def ttt_linear_fullbatch_bwd(K, Q, V, W0, eta, dZ, *, saved=None, dK=None, dQ=None, dV=None,
                             dW0=None, deta=None, loss: int = LOSS_L2):
    """Backward of ttt_linear_fullbatch for L = sum(dZ * Z).

    Returns (dK, dQ, dV, dW0, deta); dW0 [H,64,64] and deta [H] are float32
    sums over the batch.
    """
    B, H, N, d = K.shape
    _param(W0, (H, d, d), "W0")
    _param(eta, (H,), "eta")
    mk = lambda: torch.empty((B, H, N, d), dtype=K.dtype, device=K.device)
    dK = mk() if dK is None else dK
    dQ = mk() if dQ is None else dQ
    dV = mk() if dV is None else dV
    dW0 = torch.empty((H, d, d), dtype=torch.float32, device=K.device) if dW0 is None else dW0
    deta = torch.empty((H,), dtype=torch.float32, device=K.device) if deta is None else deta
    p = problem(K, loss=loss)
    ws, wsb = workspace(OP_LINEAR_FULLBATCH_BWD, p, K.device)
    st = lib().ttt_linear_fullbatch_bwd(ctypes.byref(p), view(K), view(Q), view(V), W0.data_ptr(),
                                        eta.data_ptr(), view(dZ), _ptr(saved), view(dK), view(dQ),
                                        view(dV), dW0.data_ptr(), deta.data_ptr(), ws, wsb,
                                        _stream(K.device))
    _check(st, "ttt_linear_fullbatch_bwd")
    return dK, dQ, dV, dW0, deta


def ttt_dwconv3x3_fullbatch_bwd(K, Q, V, w0, eta, dZ, grid_h: int, grid_w: int, *, saved=None, dK=None,
                                dQ=None, dV=None, dw0=None, deta=None, loss: int = LOSS_L2):
    """Backward of ttt_dwconv3x3_fullbatch for L = sum(dZ * Z).

    saved: the forward's g (float32 [B,H,64,3,3]) or None to recompute it.
    Returns (dK, dQ, dV, dw0, deta); dw0 [H,64,3,3] and deta [H] are float32
    sums over the batch.
    """
    B, H, N, d = K.shape
    _param(w0, (H, d, 3, 3), "w0")
    _param(eta, (H,), "eta")
    mk = lambda: torch.empty((B, H, N, d), dtype=K.dtype, device=K.device)
    dK = mk() if dK is None else dK
    dQ = mk() if dQ is None else dQ
    dV = mk() if dV is None else dV
    dw0 = torch.empty((H, d, 3, 3), dtype=torch.float32, device=K.device) if dw0 is None else dw0
    deta = torch.empty((H,), dtype=torch.float32, device=K.device) if deta is None else deta
    p = problem(K, grid=(grid_h, grid_w), loss=loss)
    ws, wsb = workspace(OP_DWCONV3X3_FULLBATCH_BWD, p, K.device)
    st = lib().ttt_dwconv3x3_fullbatch_bwd(ctypes.byref(p), view(K), view(Q), view(V), w0.data_ptr(),
                                           eta.data_ptr(), view(dZ), _ptr(saved), view(dK), view(dQ),
                                           view(dV), dw0.data_ptr(), deta.data_ptr(), ws, wsb,
                                           _stream(K.device))
    _check(st, "ttt_dwconv3x3_fullbatch_bwd")
    return dK, dQ, dV, dw0, deta


def ttt_linear_gradient_magnitude(K, V, W0, *, out=None, loss: int = LOSS_L2):
    """Per-token ||G_t||_F at W0 (the gradient magnitude map), float32 [B,H,N]."""
    B, H, N, d = K.shape
    _param(W0, (H, d, d), "W0")
    if out is None:
        out = torch.empty((B, H, N), dtype=torch.float32, device=K.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of shape (B, H, N)")
    p = problem(K, loss=loss)
    st = lib().ttt_linear_gradient_magnitude(ctypes.byref(p), view(K), view(V), W0.data_ptr(), out.data_ptr(),
                                             _stream(K.device))
    _check(st, "ttt_linear_gradient_magnitude")
    return out


def ttt_linear_minibatch_bidir_bwd(K, Q, V, W0, eta, dZ, minibatch: int, mode: int = BIDIR_AVG, *, dK=None,
                                   dQ=None, dV=None, dW0=None, deta=None):
    """Backward of ttt_linear_minibatch_bidir for L = sum(dZ * Z).

    W0 [H,64,64] (shared) or [2,H,64,64] (one per direction; dW0 then has
    the same shape).  Returns (dK, dQ, dV, dW0, deta)."""
    B, H, N, d = K.shape
    w0dir = 1 if W0.dim() == 4 else 0
    wshape = (2, H, d, d) if w0dir else (H, d, d)
    _param(W0, wshape, "W0")
    _param(eta, (H,), "eta")
    mk = lambda: torch.empty((B, H, N, d), dtype=K.dtype, device=K.device)
    dK = mk() if dK is None else dK
    dQ = mk() if dQ is None else dQ
    dV = mk() if dV is None else dV
    dW0 = torch.empty(wshape, dtype=torch.float32, device=K.device) if dW0 is None else dW0
    deta = torch.empty((H,), dtype=torch.float32, device=K.device) if deta is None else deta
    p = problem(K, minibatch=minibatch, mode=mode, w0_per_direction=w0dir)
    ws, wsb = workspace(OP_LINEAR_MINIBATCH_BIDIR_BWD, p, K.device)
    st = lib().ttt_linear_minibatch_bidir_bwd(ctypes.byref(p), view(K), view(Q), view(V), W0.data_ptr(),
                                              eta.data_ptr(), view(dZ), view(dK), view(dQ), view(dV),
                                              dW0.data_ptr(), deta.data_ptr(), ws, wsb, _stream(K.device))
    _check(st, "ttt_linear_minibatch_bidir_bwd")
    return dK, dQ, dV, dW0, deta


def ttt_mlp_fullbatch(K, Q, V, W1, W2, eta, *, Z=None):
    """Two-layer SiLU MLP inner model: one full-batch L2 step from (W1, W2),
    then Z = W2' silu(W1' Q).  W1 float32 [H, hidden, 64], W2 float32
    [H, 64, hidden], hidden in {64, 128, 192, 256}; bf16 views."""
    B, H, N, d = K.shape
    hid = W1.shape[1] if W1.dim() == 3 else -1
    _param(W1, (H, hid, d), "W1")
    _param(W2, (H, d, hid), "W2")
    _param(eta, (H,), "eta")
    Z = torch.empty_like(K) if Z is None else Z
    p = problem(K, hidden=hid)
    ws, wsb = workspace(OP_MLP_FULLBATCH, p, K.device)
    st = lib().ttt_mlp_fullbatch(ctypes.byref(p), view(K), view(Q), view(V), W1.data_ptr(), W2.data_ptr(),
                                 eta.data_ptr(), view(Z), ws, wsb, _stream(K.device))
    _check(st, "ttt_mlp_fullbatch")
    return Z
