"""Python binding of the cross-entropy over given logits (include/chunked_ce.h).

``chunked_ce_workspace_size``, ``chunked_ce_forward``, ``chunked_ce_backward``
and ``chunked_ce_mask_labels`` keep the C names; they check and marshal torch
device tensors and raise on a non-zero status.  ``ChunkedCrossEntropy`` and
``compute_cross_entropy`` wrap them in an autograd function with the
constructor and ``forward`` arguments of the page
"nemo_automodel.components.loss.chunked_ce".  torch supplies device memory and
the stream only; all arithmetic runs in the HIP library.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from .flce import _need, _ptr, _raise_for, _stream_ptr, raise_for_device_status

_REDUCTIONS = {"sum": _lib.FLCE_REDUCTION_SUM, "mean": _lib.FLCE_REDUCTION_MEAN}
_DTYPES = {torch.bfloat16: _lib.FLCE_DTYPE_BF16, torch.float32: _lib.FLCE_DTYPE_FP32}
_MASK_BYTES = {torch.bool: 1, torch.uint8: 1, torch.int8: 1, torch.int16: 2, torch.int32: 4, torch.int64: 8}


def make_ce_problem(num_tokens: int, vocab: int, dtype=torch.bfloat16, ignore_index: int = -100,
                    reduction: str = "sum", num_label_tokens: int | None = None,
                    chunk_len: int = 32) -> _lib.CEProblem:
    """Fill a ``chunked_ce_problem_t``; value checks are the library's."""
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_REDUCTIONS)}, got {reduction!r}")
    if dtype not in _DTYPES:
        raise NotImplementedError(f"logits must be bfloat16 or float32, got {dtype}")
    if num_label_tokens is not None and int(num_label_tokens) < 0:
        raise ValueError("num_label_tokens must be positive")
    return _lib.CEProblem(num_tokens=int(num_tokens), vocab=int(vocab), ignore_index=int(ignore_index),
                          reduction=_REDUCTIONS[reduction],
                          num_label_tokens=-1 if num_label_tokens is None else int(num_label_tokens),
                          logits_dtype=_DTYPES[dtype], chunk_len=int(chunk_len))


def chunked_ce_workspace_size(problem: _lib.CEProblem) -> int:
    out = ctypes.c_size_t(0)
    _raise_for(_lib.load().chunked_ce_workspace_size(ctypes.byref(problem), ctypes.byref(out)),
               "chunked_ce_workspace_size")
    return int(out.value)


def alloc_ce_workspace(problem: _lib.CEProblem, device) -> torch.Tensor:
    return torch.empty(max(chunked_ce_workspace_size(problem), 1), dtype=torch.uint8, device=device)


def _mask_arg(mask, T, device):
    """(tensor, element bytes) for the C call; a floating mask becomes bool
    (nonzero entries count)."""
    if mask is None:
        return None, 0
    m = mask.reshape(-1)
    if m.numel() != T:
        raise ValueError("mask must have one entry per position")
    if m.dtype.is_floating_point:
        m = m != 0
    if m.dtype not in _MASK_BYTES:
        raise ValueError(f"unsupported mask dtype {mask.dtype}")
    if m.device != device:
        raise ValueError(f"mask must be on {device}")
    return m.contiguous(), _MASK_BYTES[m.dtype]


def chunked_ce_forward(problem, logits, labels, loss, lse, mask=None, token_loss=None, device_status=None,
                       workspace=None, stream=None) -> None:
    """Enqueue the forward pass; see include/chunked_ce.h for the contract."""
    T, V = problem.num_tokens, problem.vocab
    dev = logits.device
    dtype = {v: k for k, v in _DTYPES.items()}[problem.logits_dtype]
    _need(logits, "logits", dtype, (T, V), dev)
    _need(labels, "labels", torch.int64, (T,), dev)
    _need(loss, "loss", torch.float32, (), dev)
    _need(lse, "lse", torch.float32, (T,), dev)
    if token_loss is not None:
        _need(token_loss, "token_loss", torch.float32, (T,), dev)
    if device_status is not None:
        _need(device_status, "device_status", torch.int32, (), dev)
    m, mb = _mask_arg(mask, T, dev)
    if workspace is None:
        workspace = alloc_ce_workspace(problem, dev)
    code = _lib.load().chunked_ce_forward(
        ctypes.byref(problem), _ptr(logits), _ptr(labels), _ptr(m), mb, _ptr(loss), _ptr(lse), _ptr(token_loss),
        _ptr(device_status), _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    _raise_for(code, "chunked_ce_forward")


def chunked_ce_backward(problem, logits, labels, lse, grad_out, d_logits, mask=None, device_status=None,
                        workspace=None, stream=None) -> None:
    """Enqueue the backward pass; see include/chunked_ce.h for the contract."""
    T, V = problem.num_tokens, problem.vocab
    dev = logits.device
    dtype = {v: k for k, v in _DTYPES.items()}[problem.logits_dtype]
    _need(logits, "logits", dtype, (T, V), dev)
    _need(labels, "labels", torch.int64, (T,), dev)
    _need(lse, "lse", torch.float32, (T,), dev)
    _need(grad_out, "grad_out", torch.float32, (), dev)
    _need(d_logits, "d_logits", dtype, (T, V), dev)
    if device_status is not None:
        _need(device_status, "device_status", torch.int32, (), dev)
    m, mb = _mask_arg(mask, T, dev)
    if workspace is None:
        workspace = alloc_ce_workspace(problem, dev)
    code = _lib.load().chunked_ce_backward(
        ctypes.byref(problem), _ptr(logits), _ptr(labels), _ptr(m), mb, _ptr(lse), _ptr(grad_out),
        _ptr(d_logits), _ptr(device_status), _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    _raise_for(code, "chunked_ce_backward")


def chunked_ce_mask_labels(labels, mask, ignore_index: int = -100, stream=None) -> None:
    """labels[t] = ignore_index wherever mask[t] == 0, in place, on the device."""
    if labels.dtype != torch.int64 or not labels.is_contiguous():
        raise ValueError("labels must be a contiguous int64 tensor")
    m, mb = _mask_arg(mask, labels.numel(), labels.device)
    code = _lib.load().chunked_ce_mask_labels(_ptr(labels), _ptr(m), mb, labels.numel(), int(ignore_index),
                                              _stream_ptr(stream))
    _raise_for(code, "chunked_ce_mask_labels")


class _ChunkedCE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits2d, labels1d, ignore_index, reduction, num_label_tokens, chunk_len, check_labels):
        T, V = logits2d.shape
        problem = make_ce_problem(T, V, logits2d.dtype, ignore_index, reduction, num_label_tokens, chunk_len)
        dev = logits2d.device
        ws = alloc_ce_workspace(problem, dev)
        loss = torch.empty((), dtype=torch.float32, device=dev)
        lse = torch.empty(T, dtype=torch.float32, device=dev)
        status = torch.zeros((), dtype=torch.int32, device=dev) if check_labels else None
        chunked_ce_forward(problem, logits2d, labels1d, loss, lse, device_status=status, workspace=ws)
        if check_labels:
            raise_for_device_status(status, "cross entropy")
        ctx.save_for_backward(logits2d, labels1d, lse)
        ctx.problem = problem
        return loss

    @staticmethod
    def backward(ctx, grad_out):
        logits2d, labels1d, lse = ctx.saved_tensors
        g = grad_out.detach().to(torch.float32).contiguous()
        d = torch.empty_like(logits2d)
        chunked_ce_backward(ctx.problem, logits2d, labels1d, lse, g, d)
        return d, None, None, None, None, None, None


def _apply(logits, labels, mask, ignore_index, reduction, num_label_tokens, chunk_len, check_labels=True):
    if logits.dim() < 1:
        raise ValueError("logits must have a vocabulary dimension")
    V = logits.shape[-1]
    if tuple(labels.shape) != tuple(logits.shape[:-1]):
        raise ValueError("labels must match logits.shape[:-1]")
    lab = labels.reshape(-1)
    if mask is not None:
        if tuple(mask.shape) != tuple(labels.shape):
            raise ValueError("mask must match labels' shape")
        # The page: with a mask, ignored positions are replaced with
        # ignore_index in the labels tensor.
        if lab.dtype == torch.int64 and lab.is_contiguous() and lab.data_ptr() == labels.data_ptr():
            chunked_ce_mask_labels(lab, mask, ignore_index)
        else:
            lab64 = lab.to(torch.int64).contiguous()
            chunked_ce_mask_labels(lab64, mask, ignore_index)
            labels.copy_(lab64.view(labels.shape))
            lab = lab64
    if lab.dtype != torch.int64:
        lab = lab.to(torch.int64)
    return _ChunkedCE.apply(logits.reshape(-1, V).contiguous(), lab.contiguous(), int(ignore_index), reduction,
                            num_label_tokens, int(chunk_len), bool(check_labels))


def compute_cross_entropy(logits, targets, ignore_index=-100, reduction="sum", check_labels=True):
    """Cross-entropy of ``logits`` (sequence, classes) against ``targets``
    (sequence,); the sum of the per-position losses for 'sum'.  A target
    outside [0, classes) that is not ignore_index raises ValueError unless
    ``check_labels`` is off (then it is skipped like an ignored one)."""
    return _apply(logits, targets, None, ignore_index, reduction, None, 32, check_labels)


class ChunkedCrossEntropy(torch.nn.Module):
    """Cross-entropy over given logits, with the constructor (chunk_len,
    compile, ignore_index, reduction) and ``forward`` (logits, labels, mask,
    num_label_tokens) of the chunked_ce page.

    ``chunk_len`` must be positive; the kernels never hold an fp32 copy of the
    logits, so it bounds nothing further.  ``compile`` is accepted for the
    signature: the kernels are compiled ahead of time.  ``check_labels``
    (default on) raises ValueError for a kept label outside [0, vocab) that
    is not ignore_index (one host read per forward).
    """

    def __init__(self, chunk_len: int = 32, compile: bool = True, ignore_index: int = -100,
                 reduction: str = "sum", check_labels: bool = True):
        super().__init__()
        if int(chunk_len) <= 0:
            raise ValueError("chunk_len must be positive")
        if reduction not in _REDUCTIONS:
            raise ValueError(f"reduction must be one of {sorted(_REDUCTIONS)}")
        self.chunk_len = int(chunk_len)
        self.compile = bool(compile)
        self.ignore_index = ignore_index
        self.reduction = reduction
        self.check_labels = bool(check_labels)

    def forward(self, logits, labels, mask=None, num_label_tokens=None):
        return _apply(logits, labels, mask, self.ignore_index, self.reduction, num_label_tokens, self.chunk_len,
                      self.check_labels)
