"""Fused linear cross-entropy, and cross-entropy over given logits, for AMD
MI355X (gfx950): HIP kernels behind a C ABI (include/flce.h,
include/chunked_ce.h) and a thin Python binding."""
from .chunked_ce import (  # noqa: F401
    ChunkedCrossEntropy,
    alloc_ce_workspace,
    chunked_ce_backward,
    chunked_ce_forward,
    chunked_ce_mask_labels,
    chunked_ce_workspace_size,
    compute_cross_entropy,
    make_ce_problem,
)
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
    "ChunkedCrossEntropy",
    "alloc_ce_workspace",
    "chunked_ce_backward",
    "chunked_ce_forward",
    "chunked_ce_mask_labels",
    "chunked_ce_workspace_size",
    "compute_cross_entropy",
    "make_ce_problem",
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
