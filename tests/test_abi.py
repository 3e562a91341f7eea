"""The C-ABI library on the host, no GPU: it loads, exports every symbol
include/ttt.h declares, sizes workspaces, and rejects each class of bad
argument with its status code before any HIP call (fake device addresses
are never dereferenced on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

import vision_test_sequence_amd as vt
from vision_test_sequence_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

MB = 1 << 20
BASE = 0x7f0000000000  # fake, 16-byte aligned device addresses, 64 MiB apart


def addr(i):
    return BASE + i * 64 * MB


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ttt_status|size_t|const char\*)\s+(ttt_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for f in ("ttt_linear_fullbatch", "ttt_dwconv3x3_fullbatch", "ttt_linear_minibatch_bidir",
              "ttt_linear_fullbatch_bwd", "ttt_workspace_size", "ttt_status_string"):
        assert f in names


def test_library_exports_every_declared_symbol():
    L = vt.lib()
    for f in declared_functions():
        assert hasattr(L, f), f
    out = subprocess.run(["nm", "-D", "--defined-only", vt.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ttt_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings():
    L = vt.lib()
    for i, n in enumerate(bd.STATUS_NAMES):
        assert L.ttt_status_string(i).decode() == n


def P(B=2, H=3, N=100, d=64, dtype=bd.TTT_BF16, gh=10, gw=10, b=16, mode=0):
    return bd.Problem(B, H, N, d, dtype, gh, gw, b, mode)


def V(i, B=2, H=3, N=100, d=64):
    return bd.View(addr(i), H * N * d, N * d, d)


def lin(p, K=None, Q=None, Vv=None, W0=addr(10), eta=addr(11), Z=None, saved=None,
        ws=None, wsb=None):
    L = vt.lib()
    K = K or V(0, p.B, p.H, p.N)
    Q = Q or V(1, p.B, p.H, p.N)
    Vv = Vv or V(2, p.B, p.H, p.N)
    Z = Z or V(3, p.B, p.H, p.N)
    need = L.ttt_workspace_size(bd.OP_LINEAR_FULLBATCH, ctypes.byref(p))
    if ws is None:
        ws = addr(20) if need else None
    if wsb is None:
        wsb = need
    return L.ttt_linear_fullbatch(ctypes.byref(p), K, Q, Vv, W0, eta, Z, saved, ws, wsb, None)


def test_workspace_sizes():
    L = vt.lib()
    ws = lambda op, p: L.ttt_workspace_size(op, ctypes.byref(p))
    # large single slice is split over workgroups: it needs partials
    assert ws(bd.OP_LINEAR_FULLBATCH, P(B=8, H=2, N=6084)) > 0
    # many short slices run one workgroup each: no workspace
    assert ws(bd.OP_LINEAR_FULLBATCH, P(B=128, H=2, N=196)) == 0
    assert ws(bd.OP_LINEAR_FULLBATCH, P(N=0)) == 0
    assert ws(bd.OP_LINEAR_FULLBATCH, P(d=32)) == 0
    assert ws(bd.OP_DWCONV3X3_FULLBATCH, P(N=99)) == 0  # grid mismatch
    assert L.ttt_workspace_size(0, None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), "TTT_ERR_BAD_SHAPE"),
    (dict(N=-5), "TTT_ERR_BAD_SHAPE"),
    (dict(B=-1), "TTT_ERR_BAD_SHAPE"),
    (dict(d=0), "TTT_ERR_BAD_SHAPE"),
    (dict(d=32), "TTT_ERR_UNSUPPORTED"),
    (dict(dtype=7), "TTT_ERR_UNSUPPORTED"),
])
def test_linear_shape_errors(kw, code):
    assert bd.STATUS_NAMES[lin(P(**kw))] == code


def test_empty_batch_is_ok_without_launch():
    assert lin(P(B=0)) == 0
    assert lin(P(H=0)) == 0


def test_null_pointers():
    L = vt.lib()
    p = P()
    assert bd.STATUS_NAMES[L.ttt_linear_fullbatch(None, V(0), V(1), V(2), addr(10), addr(11), V(3),
                                                  None, None, 0, None)] == "TTT_ERR_NULL_POINTER"
    assert bd.STATUS_NAMES[lin(p, K=bd.View(None, 1, 1, 64))] == "TTT_ERR_NULL_POINTER"
    assert bd.STATUS_NAMES[lin(p, W0=None)] == "TTT_ERR_NULL_POINTER"
    assert bd.STATUS_NAMES[lin(p, eta=None)] == "TTT_ERR_NULL_POINTER"


def test_bad_strides():
    p = P()
    assert bd.STATUS_NAMES[lin(p, K=bd.View(addr(0), -64, 6400, 64))] == "TTT_ERR_BAD_STRIDE"
    # two tokens on top of each other
    assert bd.STATUS_NAMES[lin(p, K=bd.View(addr(0), 3 * 100 * 64, 100 * 64, 32))] == "TTT_ERR_BAD_STRIDE"
    # heads overlapping
    assert bd.STATUS_NAMES[lin(p, K=bd.View(addr(0), 3 * 100 * 64, 50 * 64, 64))] == "TTT_ERR_BAD_STRIDE"
    # token-major [B,N,H,d] is fine
    assert lin(P(B=0), K=bd.View(addr(0), 100 * 3 * 64, 64, 3 * 64)) == 0


def test_misalignment():
    p = P()
    assert bd.STATUS_NAMES[lin(p, K=bd.View(addr(0) + 8, 3 * 100 * 64, 100 * 64, 64))] == "TTT_ERR_MISALIGNED"
    assert bd.STATUS_NAMES[lin(p, K=bd.View(addr(0), 3 * 100 * 72, 100 * 72, 68))] == "TTT_ERR_MISALIGNED"
    assert bd.STATUS_NAMES[lin(p, W0=addr(10) + 4)] == "TTT_ERR_MISALIGNED"
    assert bd.STATUS_NAMES[lin(p, eta=addr(11) + 2)] == "TTT_ERR_MISALIGNED"


def test_aliasing():
    p = P()
    # Z on top of K
    assert bd.STATUS_NAMES[lin(p, Z=V(0))] == "TTT_ERR_ALIASING"
    # saved overlapping Z
    assert bd.STATUS_NAMES[lin(p, saved=addr(3) + 4096)] == "TTT_ERR_ALIASING"
    # saved overlapping W0
    assert bd.STATUS_NAMES[lin(p, saved=addr(10))] == "TTT_ERR_ALIASING"


def test_q_may_alias_k():
    # only checks validation passes up to the workspace test
    p = P(B=8, H=2, N=6084)
    assert bd.STATUS_NAMES[lin(p, K=V(0, 8, 2, 6084), Q=V(0, 8, 2, 6084), wsb=0)] == \
        "TTT_ERR_WORKSPACE_TOO_SMALL"


def test_workspace_errors():
    p = P(B=8, H=2, N=6084)
    assert bd.STATUS_NAMES[lin(p, wsb=100)] == "TTT_ERR_WORKSPACE_TOO_SMALL"
    L = vt.lib()
    need = L.ttt_workspace_size(bd.OP_LINEAR_FULLBATCH, ctypes.byref(p))
    assert bd.STATUS_NAMES[lin(p, ws=0, wsb=need)] == "TTT_ERR_NULL_POINTER"
    # workspace overlapping an input
    assert bd.STATUS_NAMES[lin(p, ws=addr(0), wsb=need)] == "TTT_ERR_ALIASING"


def conv(p, **kw):
    L = vt.lib()
    need = L.ttt_workspace_size(bd.OP_DWCONV3X3_FULLBATCH, ctypes.byref(p))
    return L.ttt_dwconv3x3_fullbatch(ctypes.byref(p), V(0, p.B, p.H, p.N), V(1, p.B, p.H, p.N),
                                     V(2, p.B, p.H, p.N), kw.get("w0", addr(10)), addr(11),
                                     kw.get("Z", V(3, p.B, p.H, p.N)), kw.get("saved"),
                                     addr(20) if need else None, kw.get("wsb", need), None)


def test_conv_errors():
    assert bd.STATUS_NAMES[conv(P(gh=9, gw=10))] == "TTT_ERR_BAD_SHAPE"
    assert bd.STATUS_NAMES[conv(P(gh=0, gw=10))] == "TTT_ERR_BAD_SHAPE"
    assert bd.STATUS_NAMES[conv(P(), w0=None)] == "TTT_ERR_NULL_POINTER"
    assert bd.STATUS_NAMES[conv(P(), Z=V(1))] == "TTT_ERR_ALIASING"
    assert bd.STATUS_NAMES[conv(P(), saved=addr(2))] == "TTT_ERR_ALIASING"
    assert conv(P(B=0)) == 0


def scan(p, **kw):
    L = vt.lib()
    need = L.ttt_workspace_size(bd.OP_LINEAR_MINIBATCH_BIDIR, ctypes.byref(p))
    return L.ttt_linear_minibatch_bidir(ctypes.byref(p), V(0, p.B, p.H, p.N), V(1, p.B, p.H, p.N),
                                        V(2, p.B, p.H, p.N), addr(10), addr(11),
                                        kw.get("Z", V(3, p.B, p.H, p.N)),
                                        addr(20) if need else None, kw.get("wsb", need), None)


def test_scan_errors():
    assert bd.STATUS_NAMES[scan(P(b=0))] == "TTT_ERR_BAD_SHAPE"
    assert bd.STATUS_NAMES[scan(P(mode=3))] == "TTT_ERR_UNSUPPORTED"
    L = vt.lib()
    need = L.ttt_workspace_size(bd.OP_LINEAR_MINIBATCH_BIDIR, ctypes.byref(P()))
    assert bd.STATUS_NAMES[scan(P(), wsb=need - 1)] == "TTT_ERR_WORKSPACE_TOO_SMALL"
    # the averaged scan keeps one fp32 output per token, channel and direction
    one = L.ttt_workspace_size(bd.OP_LINEAR_MINIBATCH_BIDIR, ctypes.byref(P(mode=1)))
    assert need - one >= 2 * 2 * 3 * 100 * 64 * 4
    assert bd.STATUS_NAMES[scan(P(), Z=V(2))] == "TTT_ERR_ALIASING"
    # a slice's rows must be addressable with 31-bit offsets, overrun included
    # (the workspace is withheld, so a missed check could not launch)
    sn = 1 << 22
    far = bd.View(addr(3), 3 * 100 * sn, 100 * sn, sn)
    assert bd.STATUS_NAMES[scan(P(), Z=far, wsb=0)] == "TTT_ERR_UNSUPPORTED"
    assert scan(P(B=0)) == 0


def bwd(p, **kw):
    L = vt.lib()
    need = L.ttt_workspace_size(bd.OP_LINEAR_FULLBATCH_BWD, ctypes.byref(p))
    g = lambda n, i: kw.get(n, V(i, p.B, p.H, p.N))
    return L.ttt_linear_fullbatch_bwd(ctypes.byref(p), g("K", 0), g("Q", 1), g("V", 2), addr(10),
                                      addr(11), g("dZ", 4), kw.get("saved"), g("dK", 5), g("dQ", 6),
                                      g("dV", 7), kw.get("dW0", addr(12)), kw.get("deta", addr(13)),
                                      addr(20) if need else None, kw.get("wsb", need), None)


def test_bwd_errors():
    assert bd.STATUS_NAMES[bwd(P(N=0))] == "TTT_ERR_BAD_SHAPE"
    assert bd.STATUS_NAMES[bwd(P(), dK=V(0))] == "TTT_ERR_ALIASING"
    assert bd.STATUS_NAMES[bwd(P(), dQ=V(5))] == "TTT_ERR_ALIASING"
    assert bd.STATUS_NAMES[bwd(P(), dW0=addr(10))] == "TTT_ERR_ALIASING"
    assert bd.STATUS_NAMES[bwd(P(), dW0=None)] == "TTT_ERR_NULL_POINTER"
    assert bd.STATUS_NAMES[bwd(P(), saved=addr(7))] == "TTT_ERR_ALIASING"
    L = vt.lib()
    need = L.ttt_workspace_size(bd.OP_LINEAR_FULLBATCH_BWD, ctypes.byref(P()))
    # per-slice dW1 shares, dW1 and M, dW0 and deta terms, recomputed A and G
    assert need >= 2 * 3 * (8192 + 4096 + 8192 + 4096) * 4
    assert bd.STATUS_NAMES[bwd(P(), wsb=need - 1)] == "TTT_ERR_WORKSPACE_TOO_SMALL"
    assert bwd(P(B=0)) == 0


def test_python_binding_rejects_bad_params_before_the_library():
    import torch
    K = torch.zeros(1, 1, 16, 64)
    with pytest.raises(ValueError):
        vt.ttt_linear_fullbatch(K, K, K, torch.zeros(1, 64, 32), torch.ones(1))


def layer(pl, pc, Zl=None, Zc=None, Kc=None, wsb=None):
    L = vt.lib()
    need = L.ttt_layer_workspace_size(ctypes.byref(pl), ctypes.byref(pc))
    return L.ttt_layer_fullbatch(ctypes.byref(pl), V(0, pl.B, pl.H, pl.N), V(1, pl.B, pl.H, pl.N),
                                 V(2, pl.B, pl.H, pl.N), addr(10), addr(11), Zl or V(3, pl.B, pl.H, pl.N),
                                 ctypes.byref(pc), Kc or V(4, pc.B, pc.H, pc.N), V(5, pc.B, pc.H, pc.N),
                                 V(6, pc.B, pc.H, pc.N), addr(12), addr(13), Zc or V(7, pc.B, pc.H, pc.N),
                                 addr(20) if need else None, need if wsb is None else wsb, None)


def test_layer_workspace_size():
    L = vt.lib()
    pl, pc = P(B=8, H=2, N=6084, gh=78, gw=78), P(B=8, H=1, N=6084, gh=78, gw=78)
    lw = L.ttt_workspace_size(bd.OP_LINEAR_FULLBATCH, ctypes.byref(pl))
    cw = L.ttt_workspace_size(bd.OP_DWCONV3X3_FULLBATCH, ctypes.byref(pc))
    assert lw > 0 and cw > 0
    C = 256 * 64 * 4  # one counter block
    al = lambda n: (n + 255) // 256 * 256
    assert L.ttt_layer_workspace_size(ctypes.byref(pl), ctypes.byref(pc)) == C + al(lw) + cw - C
    # no linear workspace: its counter block is still reserved
    p0 = P(B=128, H=2, N=196, gh=14, gw=14)
    assert L.ttt_workspace_size(bd.OP_LINEAR_FULLBATCH, ctypes.byref(p0)) == 0
    c1 = P(B=2, H=1, N=100)
    cw1 = L.ttt_workspace_size(bd.OP_DWCONV3X3_FULLBATCH, ctypes.byref(c1))
    assert L.ttt_layer_workspace_size(ctypes.byref(p0), ctypes.byref(c1)) == C + C + cw1 - C


def test_layer_errors():
    pl, pc = P(B=2, H=2, N=100), P(B=2, H=1, N=100)
    assert bd.STATUS_NAMES[layer(pl, P(B=2, H=1, N=100, gh=9, gw=10))] == "TTT_ERR_BAD_SHAPE"
    assert layer(P(B=0, H=2, N=100), P(B=0, H=1, N=100)) == 0
    # the conv output on top of a linear input
    assert bd.STATUS_NAMES[layer(pl, pc, Zc=V(0, 2, 1, 100))] == "TTT_ERR_ALIASING"
    # the two outputs as overlapping head ranges of one [2, 3, 100, 64] tensor
    z3 = lambda h0: bd.View(addr(3) + h0 * 100 * 64 * 2, 3 * 100 * 64, 100 * 64, 64)
    assert bd.STATUS_NAMES[layer(pl, pc, Zl=z3(0), Zc=z3(1))] == "TTT_ERR_ALIASING"
    assert bd.STATUS_NAMES[layer(pl, pc, Zl=z3(1), Zc=z3(2))] == "TTT_ERR_ALIASING"
    assert bd.STATUS_NAMES[layer(pl, pc, wsb=0)] == "TTT_ERR_WORKSPACE_TOO_SMALL"
    # (disjoint head ranges of one output tensor are accepted: the GPU
    # layer tests run them; no case here may pass validation, which would
    # launch on the fake addresses)


def test_plan_and_workspace_query_errors():
    L = vt.lib()
    info = bd.PlanInfo()
    p = P(B=8, H=2, N=6084)
    assert L.ttt_plan_query(bd.OP_LINEAR_FULLBATCH, ctypes.byref(p), 0, None) == 1      # NULL_POINTER
    assert L.ttt_plan_query(bd.OP_LINEAR_FULLBATCH, None, 0, ctypes.byref(info)) == 1
    assert L.ttt_plan_query(bd.OP_LINEAR_FULLBATCH, ctypes.byref(P(N=0)), 0, ctypes.byref(info)) == 2
    assert L.ttt_plan_query(bd.OP_LINEAR_MINIBATCH_BIDIR, ctypes.byref(p), 0, ctypes.byref(info)) == 5
    assert L.ttt_plan_query(bd.OP_DWCONV3X3_FULLBATCH, ctypes.byref(P(N=100, gh=9, gw=10)), 0,
                            ctypes.byref(info)) == 2
    # an empty batch plans nothing
    assert L.ttt_plan_query(bd.OP_LINEAR_FULLBATCH, ctypes.byref(P(B=0)), 0, ctypes.byref(info)) == 0
    assert (info.kernel, info.splits) == (0, 0)
    # on any device (or none) a plan names one of the kernels
    assert L.ttt_plan_query(bd.OP_LINEAR_FULLBATCH, ctypes.byref(p), 0, ctypes.byref(info)) == 0
    assert info.kernel in (bd.KERNEL_LIN_RESIDENT, bd.KERNEL_LIN_RESIDENT_GX, bd.KERNEL_LIN_STREAM)
    assert info.splits >= 1
    f = ctypes.c_int32(7)
    assert L.ttt_layer_plan_query(ctypes.byref(p), ctypes.byref(P(N=100)), None) == 1
    assert L.ttt_layer_plan_query(ctypes.byref(p), ctypes.byref(P(N=100, gh=9, gw=10)), ctypes.byref(f)) == 2
    # workspace queries: argument errors come before any HIP call
    assert L.ttt_workspace_exchange_failed(bd.OP_LINEAR_FULLBATCH, addr(1), 4096, None, None) == 1
    assert L.ttt_workspace_exchange_failed(bd.OP_LINEAR_FULLBATCH, None, 4096, ctypes.byref(f), None) == 1
    assert L.ttt_workspace_exchange_failed(bd.OP_LINEAR_FULLBATCH, addr(1) + 16, 4096, ctypes.byref(f), None) == 4
    assert L.ttt_workspace_exchange_failed(9, addr(1), 4096, ctypes.byref(f), None) == 5
    f.value = 7
    assert L.ttt_workspace_exchange_failed(bd.OP_LINEAR_FULLBATCH, None, 0, ctypes.byref(f), None) == 0
    assert f.value == 0
    assert L.ttt_workspace_exchange_failed(bd.OP_LINEAR_MINIBATCH_BIDIR, addr(1), 4096, ctypes.byref(f),
                                           None) == 0 and f.value == 0  # the scan has no counters
    assert L.ttt_workspace_reset(None, 0, None) == 0
    assert L.ttt_workspace_reset(None, 256, None) == 1


def test_noalloc_scratch_holds_every_linear_workspace():
    # the allocation-free entry point's fixed scratch (10.5 MiB) must hold
    # the workspace of any problem shape it accepts
    L = vt.lib()
    worst = 0
    for slices in list(range(1, 300)) + [1000, 4096, 1 << 16]:
        for N in (1, 100, 128, 129, 1000, 4096, 6084, 10000, 100000, 1 << 20, (1 << 31) - 1):
            p = P(B=slices, H=1, N=N)
            worst = max(worst, L.ttt_workspace_size(bd.OP_LINEAR_FULLBATCH, ctypes.byref(p)))
    assert 0 < worst <= 21 << 19, worst


def test_noalloc_argument_errors():
    L = vt.lib()
    p = P()
    f = L.ttt_linear_fullbatch_noalloc
    ok = dict(K=V(0), Q=V(1), Vv=V(2), Z=V(3))
    call = lambda pp=p, K=ok["K"], Q=ok["Q"], Vv=ok["Vv"], W0=addr(10), eta=addr(11), Z=ok["Z"], saved=None: \
        f(ctypes.byref(pp) if pp is not None else None, K, Q, Vv, W0, eta, Z, saved, None)
    assert call(pp=None) == 1
    assert call(pp=P(N=0)) == 2
    assert call(pp=P(d=32)) == 5
    assert call(W0=None) == 1
    assert call(K=bd.View(0, 300 * 64, 100 * 64, 64)) == 1
    assert call(W0=addr(10) + 4) == 4
    assert call(Z=V(0)) == 6                       # Z overlaps K
    assert call(saved=addr(1)) == 6                # saved overlaps Q
    assert call(pp=P(B=0)) == 0                    # empty: no launch


def test_conv_bwd_errors():
    L = vt.lib()
    p = P(B=2, H=3, N=100, gh=10, gw=10)
    need = L.ttt_workspace_size(bd.OP_DWCONV3X3_FULLBATCH_BWD, ctypes.byref(p))
    assert need > 0
    assert L.ttt_workspace_size(bd.OP_DWCONV3X3_FULLBATCH_BWD, ctypes.byref(P(N=100, gh=9, gw=10))) == 0
    f = L.ttt_dwconv3x3_fullbatch_bwd

    def call(pp=p, saved=None, dK=V(6), dQ=V(7), dV=V(8), dw0=addr(12), deta=addr(13), ws=addr(20),
             wsb=need, w0=addr(10)):
        return f(ctypes.byref(pp), V(0), V(1), V(2), w0, addr(11), V(3), saved, dK, dQ, dV, dw0, deta,
                 ws, wsb, None)
    assert call(pp=P(N=100, gh=9, gw=10)) == 2          # grid does not cover N
    assert call(pp=P(B=0, N=100, gh=10, gw=10)) == 0    # empty: no launch
    assert call(dw0=None) == 1
    assert call(w0=addr(10) + 4) == 4
    assert call(dK=V(0)) == 6                           # dK overlaps K
    assert call(dQ=V(6)) == 6                           # two outputs overlap
    assert call(saved=addr(8)) == 6                     # saved overlaps the dV output
    assert call(wsb=need - 1) == 7
    assert call(ws=addr(20) + 16) == 4
    # a slice of each view is addressed with 32-bit offsets: 100 tokens
    # 2^22 elements apart span more than 2^29 bytes (checked before any
    # launch: the workspace is withheld)
    sn = 1 << 22
    far = bd.View(addr(9), 3 * 100 * sn, 100 * sn, sn)
    assert bd.STATUS_NAMES[call(dV=far, wsb=0)] == "TTT_ERR_UNSUPPORTED"


def test_scan_bwd_errors():
    L = vt.lib()
    f = L.ttt_linear_minibatch_bidir_bwd
    p = P(b=16)
    need = L.ttt_workspace_size(bd.OP_LINEAR_MINIBATCH_BIDIR_BWD, ctypes.byref(p))
    assert need > 0
    assert L.ttt_workspace_size(bd.OP_LINEAR_MINIBATCH_BIDIR_BWD, ctypes.byref(P(b=33))) == 0

    def call(pp=p, dK=V(6), dW0=addr(12), wsb=need, W0=addr(10)):
        return f(ctypes.byref(pp), V(0), V(1), V(2), W0, addr(11), V(3), dK, V(7), V(8), dW0, addr(13),
                 addr(20), wsb, None)
    assert call(pp=P(b=0)) == 2
    assert call(pp=P(b=33)) == 5                     # more than 32 tokens per mini-batch
    assert call(pp=P(b=16, mode=3)) == 5
    assert call(pp=bd.Problem(2, 3, 100, 64, bd.TTT_BF16, 10, 10, 16, 0, bd.LOSS_DOT, 1, 0)) == 5
    assert call(pp=P(b=16, B=0)) == 0
    assert call(dW0=None) == 1
    assert call(dK=V(0)) == 6
    assert call(wsb=need - 1) == 7
    assert call(W0=addr(10) + 4) == 4


def test_mlp_errors():
    L = vt.lib()
    f = L.ttt_mlp_fullbatch

    def M(hidden=256, dtype=bd.TTT_BF16, loss=bd.LOSS_L2, steps=1, B=2, d=64):
        return bd.Problem(B, 3, 100, d, dtype, 10, 10, 0, 0, loss, steps, 0, hidden)
    p = M()
    need = L.ttt_workspace_size(bd.OP_MLP_FULLBATCH, ctypes.byref(p))
    assert need > 0
    for hid in (64, 128, 192):
        assert 0 < L.ttt_workspace_size(bd.OP_MLP_FULLBATCH, ctypes.byref(M(hidden=hid))) < need
    assert L.ttt_workspace_size(bd.OP_MLP_FULLBATCH, ctypes.byref(M(hidden=96))) == 0

    def call(pp=p, W1=addr(10), W2=addr(11), Z=V(3), wsb=need):
        return f(ctypes.byref(pp), V(0), V(1), V(2), W1, W2, addr(12), Z, addr(20), wsb, None)
    assert call(pp=M(hidden=0)) == 2
    assert call(pp=M(hidden=96)) == 5                 # widths are 64 r, r = 1..4
    assert call(pp=M(hidden=320)) == 5
    assert call(pp=M(dtype=bd.TTT_F32)) == 5          # bf16 only
    assert call(pp=M(loss=bd.LOSS_DOT)) == 5
    assert call(pp=M(steps=2)) == 5
    assert call(pp=M(d=32)) == 5
    assert call(pp=M(B=0)) == 0                       # empty: no launch
    assert call(W1=None) == 1
    assert call(W2=addr(11) + 2) == 4
    assert call(Z=V(0)) == 6                          # Z overlaps K
    assert call(W1=addr(3)) == 6                      # W1 inside Z
    assert call(wsb=need - 1) == 7
