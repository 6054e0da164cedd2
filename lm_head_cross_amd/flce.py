"""Python binding of the fused linear cross-entropy C ABI (include/flce.h).

The functions ``flce_workspace_size``, ``flce_forward`` and ``flce_backward``
keep the C names; they check and marshal torch device tensors and raise on a
non-zero status.  ``FusedLinearCrossEntropy`` and
``Inkling2FusedLinearCrossEntropy`` wrap them in an autograd function with
the constructor and ``forward`` arguments of the NeMo AutoModel pages
("nemo_automodel.components.loss.linear_ce", FusedLinearCrossEntropy;
"nemo_automodel.components.models.inkling2.loss",
Inkling2FusedLinearCrossEntropy).  torch supplies device memory and the
stream only; all arithmetic runs in the HIP library.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_REDUCTIONS = {"sum": _lib.FLCE_REDUCTION_SUM, "mean": _lib.FLCE_REDUCTION_MEAN}


class FlceError(RuntimeError):
    """A non-argument failure reported by the library (e.g. a HIP launch)."""


def _raise_for(code: int, what: str) -> None:
    if code == _lib.FLCE_OK:
        return
    msg = f"{what}: {_lib.status_string(code)} (status {code})"
    if code in (_lib.FLCE_ERR_INVALID_ARG, _lib.FLCE_ERR_WORKSPACE):
        raise ValueError(msg)
    if code == _lib.FLCE_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise FlceError(msg)


_WEIGHT_DTYPES = {torch.bfloat16: _lib.FLCE_DTYPE_BF16, torch.float32: _lib.FLCE_DTYPE_FP32}


_DW_TILE_FLAGS = {None: 0, 256: _lib.FLCE_FLAG_DW_TILE_256, 384: _lib.FLCE_FLAG_DW_TILE_384}


def make_problem(num_tokens: int, hidden: int, vocab: int, unpadded_vocab: int | None = None,
                 softcap: float = 0.0, ignore_index: int = -100, reduction: str = "sum",
                 num_label_tokens: int | None = None, weight_dtype=torch.bfloat16,
                 round_head_on_load: bool = False, dw_tile: int | None = None,
                 head_staged: bool = False) -> _lib.Problem:
    """Fill an ``flce_problem_t``; value checks are the library's.  With
    ``weight_dtype=torch.float32`` the calls take the fp32 head and round its
    usable rows to bf16 themselves: staged in the workspace, or with
    ``round_head_on_load`` inside the GEMMs' tile loads (smaller workspace,
    slower; see include/flce.h).  ``dw_tile`` (256 or 384) fixes the tile of
    the backward's dW contraction, which the library otherwise picks.
    ``head_staged``: the backward reuses the head copy that the matching
    forward staged in the same workspace (FLCE_FLAG_HEAD_STAGED; the caller
    vouches that the workspace and head are untouched in between)."""
    if weight_dtype not in _WEIGHT_DTYPES:
        raise NotImplementedError(f"the head must be bfloat16 or float32, got {weight_dtype}")
    if dw_tile not in _DW_TILE_FLAGS:
        raise ValueError(f"dw_tile must be None, 256 or 384, got {dw_tile!r}")
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_REDUCTIONS)}, got {reduction!r}")
    if num_label_tokens is not None and int(num_label_tokens) < 0:
        raise ValueError("num_label_tokens must be positive")
    return _lib.Problem(
        num_tokens=int(num_tokens), hidden=int(hidden), vocab=int(vocab),
        unpadded_vocab=int(vocab if unpadded_vocab is None else unpadded_vocab),
        softcap=float(softcap), reduction=_REDUCTIONS[reduction], ignore_index=int(ignore_index),
        num_label_tokens=-1 if num_label_tokens is None else int(num_label_tokens),
        weight_dtype=_WEIGHT_DTYPES[weight_dtype],
        flags=(_lib.FLCE_FLAG_ROUND_HEAD_ON_LOAD if round_head_on_load else 0) | _DW_TILE_FLAGS[dw_tile]
        | (_lib.FLCE_FLAG_HEAD_STAGED if head_staged else 0))


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream_ptr(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, shape, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _weight_dtype(problem):
    return {v: k for k, v in _WEIGHT_DTYPES.items()}[problem.weight_dtype]


def flce_workspace_size(problem: _lib.Problem) -> int:
    """Workspace bytes ``flce_forward`` / ``flce_backward`` need."""
    out = ctypes.c_size_t(0)
    _raise_for(_lib.load().flce_workspace_size(ctypes.byref(problem), ctypes.byref(out)),
               "flce_workspace_size")
    return int(out.value)


def flce_backward_plan(problem, cu_count: int = 0) -> tuple[int, int, int]:
    """The backward pass's plan: (chunk width in head rows, number of
    chunks, rows of the dW tiles), for ``cu_count`` compute units (0: the
    current device's); see include/flce.h."""
    rows, n, tile = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int(0)
    _raise_for(_lib.load().flce_backward_plan(ctypes.byref(problem), int(cu_count), ctypes.byref(rows),
                                              ctypes.byref(n), ctypes.byref(tile)), "flce_backward_plan")
    return rows.value, n.value, tile.value


def alloc_workspace(problem: _lib.Problem, device) -> torch.Tensor:
    return torch.empty(max(flce_workspace_size(problem), 1), dtype=torch.uint8, device=device)


def flce_forward(problem, hidden, weight, labels, loss, lse, token_loss=None, device_status=None,
                 workspace=None, stream=None) -> None:
    """Enqueue the forward pass; see include/flce.h for the contract."""
    T, H, V = problem.num_tokens, problem.hidden, problem.vocab
    dev = weight.device
    _need(weight, "weight", _weight_dtype(problem), (V, H), dev)
    _need(hidden, "hidden", torch.bfloat16, (T, H), dev)
    _need(labels, "labels", torch.int64, (T,), dev)
    _need(loss, "loss", torch.float32, (), dev)
    _need(lse, "lse", torch.float32, (T,), dev)
    if token_loss is not None:
        _need(token_loss, "token_loss", torch.float32, (T,), dev)
    if device_status is not None:
        _need(device_status, "device_status", torch.int32, (), dev)
    if workspace is None:
        workspace = alloc_workspace(problem, dev)
    code = _lib.load().flce_forward(
        ctypes.byref(problem), _ptr(hidden), _ptr(weight), _ptr(labels), _ptr(loss), _ptr(lse),
        _ptr(token_loss), _ptr(device_status), _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    _raise_for(code, "flce_forward")


def flce_forward_noalloc(problem, hidden, weight, labels, loss, lse, token_loss=None, device_status=None,
                         stream=None) -> None:
    """Enqueue the forward pass on the library's fixed per-device scratch (no
    workspace, nothing allocated); see include/flce.h for the size limit and
    the rule that calls overlapping on one device race."""
    T, H, V = problem.num_tokens, problem.hidden, problem.vocab
    dev = weight.device
    _need(weight, "weight", _weight_dtype(problem), (V, H), dev)
    _need(hidden, "hidden", torch.bfloat16, (T, H), dev)
    _need(labels, "labels", torch.int64, (T,), dev)
    _need(loss, "loss", torch.float32, (), dev)
    _need(lse, "lse", torch.float32, (T,), dev)
    if token_loss is not None:
        _need(token_loss, "token_loss", torch.float32, (T,), dev)
    if device_status is not None:
        _need(device_status, "device_status", torch.int32, (), dev)
    code = _lib.load().flce_forward_noalloc(
        ctypes.byref(problem), _ptr(hidden), _ptr(weight), _ptr(labels), _ptr(loss), _ptr(lse),
        _ptr(token_loss), _ptr(device_status), _stream_ptr(stream))
    _raise_for(code, "flce_forward_noalloc")


def flce_backward(problem, hidden, weight, labels, lse, grad_out, d_hidden, d_weight, device_status=None,
                  workspace=None, stream=None) -> None:
    """Enqueue the backward pass; see include/flce.h for the contract."""
    T, H, V = problem.num_tokens, problem.hidden, problem.vocab
    dev = weight.device
    _need(weight, "weight", _weight_dtype(problem), (V, H), dev)
    _need(hidden, "hidden", torch.bfloat16, (T, H), dev)
    _need(labels, "labels", torch.int64, (T,), dev)
    _need(lse, "lse", torch.float32, (T,), dev)
    _need(grad_out, "grad_out", torch.float32, (), dev)
    _need(d_hidden, "d_hidden", torch.bfloat16, (T, H), dev)
    _need(d_weight, "d_weight", torch.float32, (V, H), dev)
    if device_status is not None:
        _need(device_status, "device_status", torch.int32, (), dev)
    if workspace is None:
        workspace = alloc_workspace(problem, dev)
    code = _lib.load().flce_backward(
        ctypes.byref(problem), _ptr(hidden), _ptr(weight), _ptr(labels), _ptr(lse), _ptr(grad_out),
        _ptr(d_hidden), _ptr(d_weight), _ptr(device_status), _ptr(workspace), workspace.numel(),
        _stream_ptr(stream))
    _raise_for(code, "flce_backward")


def flce_round_to_bf16(src: torch.Tensor, dst: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Round an fp32 tensor to bf16 (nearest, ties to even) in the library."""
    if src.dtype != torch.float32 or not src.is_contiguous():
        raise ValueError("src must be a contiguous float32 tensor")
    if dst is None:
        dst = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    _need(dst, "dst", torch.bfloat16, src.shape, src.device)
    _raise_for(_lib.load().flce_round_to_bf16(_ptr(src), _ptr(dst), src.numel(), _stream_ptr(stream)),
               "flce_round_to_bf16")
    return dst


class LaunchTrace:
    """Record the library's kernel launches with HIP events (flce_trace_*).

    ``start()`` creates the events (outside any timed region); every launch
    made until ``stop()`` is bracketed by an event pair on its stream.
    ``records()`` returns (kind name, milliseconds, algorithmic flops) per
    launch and waits for the events.
    """

    def __init__(self, capacity: int = 4096, kinds=None):
        self.capacity = capacity
        self.kinds = kinds

    def start(self):
        """Start recording; with ``kinds`` (kind names), only those kinds."""
        lib = _lib.load()
        mask = 0xFFFFFFFF
        if self.kinds is not None:
            mask = 0
            for k in self.kinds:
                mask |= 1 << _lib.KERNEL_KINDS.index(k)
        _raise_for(lib.flce_trace_select(mask), "flce_trace_select")
        _raise_for(lib.flce_trace_start(self.capacity), "flce_trace_start")
        return self

    def stop(self):
        """Stop recording; the kind filter goes back to every kind."""
        lib = _lib.load()
        lib.flce_trace_stop()
        lib.flce_trace_select(0xFFFFFFFF)

    def records(self):
        lib = _lib.load()
        out = []
        kind = ctypes.c_int(0)
        ms = ctypes.c_float(0)
        fl = ctypes.c_double(0)
        for i in range(lib.flce_trace_count()):
            _raise_for(lib.flce_trace_get(i, ctypes.byref(kind), ctypes.byref(ms), ctypes.byref(fl)),
                       "flce_trace_get")
            out.append((_lib.KERNEL_KINDS[kind.value], float(ms.value), float(fl.value)))
        return out


# ---------------------------------------------------------------------------
# Autograd and modules
# ---------------------------------------------------------------------------


def raise_for_device_status(status: torch.Tensor, what: str) -> None:
    """Raise ValueError if the device status word reports a label outside
    [0, unpadded vocabulary) that is not ignore_index (waits for the stream
    that wrote it)."""
    if int(status.item()) & _lib.FLCE_DEVICE_BAD_LABEL:
        raise ValueError(f"{what}: a label is neither ignore_index nor inside [0, unpadded vocabulary) "
                         "(PyTorch's cross entropy rejects such a target)")


class _FusedLinearCE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, labels, unpadded_vocab, softcap, ignore_index, reduction,
                num_label_tokens, check_labels):
        T, H = hidden.shape
        problem = make_problem(T, H, weight.shape[0], unpadded_vocab, softcap, ignore_index, reduction,
                               num_label_tokens)
        dev = hidden.device
        ctx.weight_dtype = weight.dtype
        if weight.dtype == torch.float32:
            weight = flce_round_to_bf16(weight)
        ws = alloc_workspace(problem, dev)
        loss = torch.empty((), dtype=torch.float32, device=dev)
        lse = torch.empty(T, dtype=torch.float32, device=dev)
        status = torch.zeros((), dtype=torch.int32, device=dev) if check_labels else None
        flce_forward(problem, hidden, weight, labels, loss, lse, device_status=status, workspace=ws)
        if check_labels:
            raise_for_device_status(status, "fused linear cross entropy")
        ctx.save_for_backward(hidden, weight, labels, lse)
        ctx.problem = problem
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        hidden, weight, labels, lse = ctx.saved_tensors
        problem = ctx.problem
        g = grad_out.detach().to(torch.float32).contiguous()
        d_hidden = torch.empty_like(hidden)
        d_weight = torch.empty(weight.shape, dtype=torch.float32, device=weight.device)
        flce_backward(problem, hidden, weight, labels, lse, g, d_hidden, d_weight)
        # The bf16 rounding of an fp32 head passes the gradient through, so
        # d_weight is already the fp32 head's gradient.
        return d_hidden, d_weight, None, None, None, None, None, None, None


def fused_linear_cross_entropy(hidden_states, labels, lm_weight, unpadded_vocab_size=None,
                               logit_softcapping=0.0, ignore_index=-100, reduction="sum",
                               num_label_tokens=None, check_labels=True):
    """Loss of ``hidden_states`` [..., H] against ``lm_weight`` [V, H].

    An fp32 head takes part through its bf16 value (round to nearest even,
    done by the library), per the Inkling2 loss page; the fp32 head receives
    the fp32 gradient.  With ``check_labels`` (the default) a label that is
    neither ignore_index nor inside the usable vocabulary raises ValueError,
    as PyTorch's cross entropy does; the check reads the library's device
    status word once, which waits for the forward pass.  With it off, such a
    position is skipped like an ignored one.
    """
    H = hidden_states.shape[-1]
    hidden = hidden_states.reshape(-1, H)
    if hidden.dtype != torch.bfloat16:
        raise ValueError("hidden_states must be bfloat16")
    if lm_weight.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("lm_weight must be bfloat16 or float32")
    w = lm_weight
    lab = labels.reshape(-1)
    if lab.numel() != hidden.shape[0]:
        raise ValueError("labels must have one entry per hidden-state position")
    if lab.dtype != torch.int64:
        lab = lab.to(torch.int64)
    return _FusedLinearCE.apply(hidden.contiguous(), w.contiguous(), lab.contiguous(),
                                unpadded_vocab_size, float(logit_softcapping), int(ignore_index),
                                reduction, num_label_tokens, bool(check_labels))


class FusedLinearCrossEntropy(torch.nn.Module):
    """Fused projection and cross-entropy over hidden states and an LM head.

    Mirrors the constructor (ignore_index, logit_softcapping, reduction) and
    ``forward`` (hidden_states, labels, lm_weight, num_label_tokens,
    grad_reduce_group) of the linear_ce page; the loss is a scalar on the
    device of ``hidden_states``.  ``unpadded_vocab_size`` (None: every head
    row) restricts the softmax to the first rows, as on the Inkling2 page.
    The head's gradient is computed in fp32 and handed to autograd, which
    gives a bf16 head a bf16 gradient and an fp32 head the fp32 one.
    ``check_labels`` (default on) raises ValueError for a label outside the
    usable vocabulary that is not ignore_index (one host read per forward).
    """

    def __init__(self, ignore_index: int = -100, logit_softcapping: float = 0, reduction: str = "sum",
                 unpadded_vocab_size: int | None = None, check_labels: bool = True):
        super().__init__()
        if reduction not in _REDUCTIONS:
            raise ValueError(f"reduction must be one of {sorted(_REDUCTIONS)}")
        if logit_softcapping < 0:
            raise ValueError("logit_softcapping must be >= 0")
        if unpadded_vocab_size is not None and unpadded_vocab_size <= 0:
            raise ValueError("unpadded_vocab_size must be positive")
        self.ignore_index = ignore_index
        self.logit_softcapping = logit_softcapping
        self.reduction = reduction
        self.unpadded_vocab_size = None if unpadded_vocab_size is None else int(unpadded_vocab_size)
        self.check_labels = bool(check_labels)

    @staticmethod
    def materialize_lm_weight(lm_weight, grad_reduce_group=None):
        """A regular tensor is returned unchanged (linear_ce page,
        materialize_lm_weight).  Sharded heads need several GPUs and are not
        supported here."""
        if type(lm_weight).__name__ == "DTensor":
            raise NotImplementedError("sharded (DTensor) LM heads are not supported on one GPU")
        return lm_weight

    def forward(self, hidden_states, labels, lm_weight, num_label_tokens=None, grad_reduce_group=None):
        if grad_reduce_group is not None:
            raise NotImplementedError("grad_reduce_group needs a sharded head across GPUs")
        w = self.materialize_lm_weight(lm_weight, grad_reduce_group)
        return fused_linear_cross_entropy(hidden_states, labels, w, self.unpadded_vocab_size,
                                          self.logit_softcapping, self.ignore_index, self.reduction,
                                          num_label_tokens, self.check_labels)


class Inkling2FusedLinearCrossEntropy(FusedLinearCrossEntropy):
    """Softcapped fused cross entropy over the first ``unpadded_vocab_size``
    head rows (Inkling2 loss page; softcap default 30)."""

    def __init__(self, unpadded_vocab_size: int, logit_softcapping: float = 30.0, ignore_index: int = -100,
                 reduction: str = "sum", check_labels: bool = True):
        if unpadded_vocab_size is None:
            raise ValueError("unpadded_vocab_size is required")
        super().__init__(ignore_index, logit_softcapping, reduction, unpadded_vocab_size, check_labels)
