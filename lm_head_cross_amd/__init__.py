"""Fused linear cross-entropy for AMD MI355X (gfx950): HIP kernels behind a
C ABI (include/flce.h) and a thin Python binding."""
from .flce import (  # noqa: F401
    FlceError,
    FusedLinearCrossEntropy,
    LaunchTrace,
    Inkling2FusedLinearCrossEntropy,
    alloc_workspace,
    flce_backward,
    flce_forward,
    flce_round_to_bf16,
    flce_workspace_size,
    fused_linear_cross_entropy,
    make_problem,
)

__all__ = [
    "FlceError",
    "FusedLinearCrossEntropy",
    "LaunchTrace",
    "Inkling2FusedLinearCrossEntropy",
    "alloc_workspace",
    "flce_backward",
    "flce_forward",
    "flce_round_to_bf16",
    "flce_workspace_size",
    "fused_linear_cross_entropy",
    "make_problem",
]
