"""MI355X (gfx950) multi-head test-time-training layer.

The compute lives in ``libttt.so`` (hand-written HIP kernels behind the C ABI
of ``include/ttt.h``); ``binding`` marshals torch tensors into that ABI and
nothing else.  There is no CPU fallback: calling an entry point without the
built library or without a GPU raises.
"""
from .binding import (  # noqa: F401
    TTT_BF16,
    TTT_F32,
    LOSS_DOT,
    LOSS_L2,
    TTTError,
    BIDIR_AVG,
    FORWARD_ONLY,
    BACKWARD_ONLY,
    exchange_failures,
    lib,
    library_path,
    plan_dwconv,
    plan_layer_fused,
    plan_linear,
    reset_workspaces,
    ttt_dwconv3x3_fullbatch,
    ttt_dwconv3x3_fullbatch_bwd,
    ttt_layer_fullbatch,
    ttt_linear_fullbatch,
    ttt_linear_fullbatch_bwd,
    ttt_linear_fullbatch_noalloc,
    ttt_linear_gradient_magnitude,
    ttt_linear_minibatch_bidir,
    ttt_linear_minibatch_bidir_bwd,
    ttt_mlp_fullbatch,
)
