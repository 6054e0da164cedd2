"""ctypes loader for ``libflce.so`` and the C structures of include/flce.h and
include/chunked_ce.h.

Argument marshalling only: every step of the computation runs in the HIP
library.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce.so")

FLCE_OK = 0
FLCE_ERR_INVALID_ARG = 1
FLCE_ERR_UNSUPPORTED = 2
FLCE_ERR_WORKSPACE = 3
FLCE_ERR_HIP = 4
FLCE_DEVICE_BAD_LABEL = 1
FLCE_REDUCTION_SUM = 0
FLCE_REDUCTION_MEAN = 1
FLCE_DTYPE_BF16 = 0
FLCE_DTYPE_FP32 = 1
FLCE_FLAG_ROUND_HEAD_ON_LOAD = 1
FLCE_FLAG_DW_TILE_256 = 2
FLCE_FLAG_DW_TILE_384 = 4
FLCE_FLAG_HEAD_STAGED = 8

EXPORTED = ("flce_status_string", "flce_version", "flce_workspace_size", "flce_backward_plan", "flce_forward",
            "flce_forward_noalloc",
            "flce_backward",
            "flce_round_to_bf16", "flce_trace_start", "flce_trace_select", "flce_trace_stop", "flce_trace_count", "flce_trace_get",
            "chunked_ce_workspace_size", "chunked_ce_forward", "chunked_ce_backward", "chunked_ce_mask_labels")

KERNEL_KINDS = ("compact", "gather", "proj_lse", "combine", "finalize", "recompute_g", "dweight", "dhidden",
                "aux", "ce_forward", "ce_backward", "dgrad")


class Problem(ctypes.Structure):
    """flce_problem_t."""

    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("unpadded_vocab", ctypes.c_int64),
        ("softcap", ctypes.c_float),
        ("reduction", ctypes.c_int32),
        ("ignore_index", ctypes.c_int64),
        ("num_label_tokens", ctypes.c_int64),
        ("weight_dtype", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class CEProblem(ctypes.Structure):
    """chunked_ce_problem_t."""

    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("ignore_index", ctypes.c_int64),
        ("reduction", ctypes.c_int32),
        ("num_label_tokens", ctypes.c_int64),
        ("logits_dtype", ctypes.c_int32),
        ("chunk_len", ctypes.c_int64),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the library once.  torch is imported first so that the library
    binds to the HIP runtime torch already loaded (same soname)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads the HIP runtime the library links against)

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m lm_head_cross_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    P = ctypes.POINTER(Problem)
    lib.flce_status_string.restype = ctypes.c_char_p
    lib.flce_status_string.argtypes = [ctypes.c_int]
    lib.flce_version.restype = ctypes.c_int
    lib.flce_version.argtypes = []
    lib.flce_workspace_size.restype = ctypes.c_int
    lib.flce_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.flce_backward_plan.restype = ctypes.c_int
    lib.flce_backward_plan.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int)]
    lib.flce_forward.restype = ctypes.c_int
    lib.flce_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.flce_forward_noalloc.restype = ctypes.c_int
    lib.flce_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.flce_backward.restype = ctypes.c_int
    lib.flce_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.flce_trace_start.restype = ctypes.c_int
    lib.flce_trace_start.argtypes = [ctypes.c_int]
    lib.flce_trace_select.restype = ctypes.c_int
    lib.flce_trace_select.argtypes = [ctypes.c_uint32]
    lib.flce_trace_stop.restype = ctypes.c_int
    lib.flce_trace_stop.argtypes = []
    lib.flce_trace_count.restype = ctypes.c_int
    lib.flce_trace_count.argtypes = []
    lib.flce_trace_get.restype = ctypes.c_int
    lib.flce_trace_get.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float),
                                   ctypes.POINTER(ctypes.c_double)]
    lib.flce_round_to_bf16.restype = ctypes.c_int
    lib.flce_round_to_bf16.argtypes = [vp, vp, ctypes.c_int64, vp]
    C = ctypes.POINTER(CEProblem)
    i32 = ctypes.c_int32
    lib.chunked_ce_workspace_size.restype = ctypes.c_int
    lib.chunked_ce_workspace_size.argtypes = [C, ctypes.POINTER(ctypes.c_size_t)]
    lib.chunked_ce_forward.restype = ctypes.c_int
    lib.chunked_ce_forward.argtypes = [C, vp, vp, vp, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.chunked_ce_backward.restype = ctypes.c_int
    lib.chunked_ce_backward.argtypes = [C, vp, vp, vp, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.chunked_ce_mask_labels.restype = ctypes.c_int
    lib.chunked_ce_mask_labels.argtypes = [vp, vp, i32, ctypes.c_int64, ctypes.c_int64, vp]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().flce_status_string(code).decode()
