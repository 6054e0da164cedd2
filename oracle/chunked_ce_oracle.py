"""Cross-entropy over given logits (the chunked CE): plain fp64 CPU oracle.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
constant or helper with that path.

What is computed, restated from the page
"nemo_automodel.components.loss.chunked_ce":

* ChunkedCrossEntropy.forward: ``logits`` has shape [..., vocab] with any
  leading token dimensions and ``labels`` the leading shape; an optional
  ``mask`` of the labels' shape marks with nonzero entries the positions that
  count, and the positions where it is zero take the ``ignore_index`` label;
  ``num_label_tokens`` is a global count dividing the sum-reduced loss; the
  result is a scalar.
* _ChunkedCrossEntropySum.forward: the sum-reduced cross-entropy, evaluated
  in fp32 a bounded number of rows (``chunk_len``) at a time from logits that
  keep their own dtype; a position whose label equals ``ignore_index`` adds
  zero loss and zero gradient.  ``chunk_len`` bounds memory only and must be
  positive (_validate_chunk_len).
* _ChunkedCrossEntropySum.backward: the softmax is recomputed and the
  gradient with respect to the logits, scaled by the scalar ``grad_out``, is
  returned.
* compute_cross_entropy: the sum of the per-position cross-entropies.

Every step is the plain definition in float64 on the exact values of the
given logits (bf16 and fp32 values are exact in float64).  The log-sum-exp,
the softmax-minus-onehot and the normaliser are the fused linear oracle's own
definitions (those of the main page's loss), applied to the logits as given.

Readings of points the page leaves open:

* reductions 'sum' and 'mean', and ``num_label_tokens`` dividing either, as
  for the fused linear loss;
* a label other than ``ignore_index`` outside [0, vocab) is an error, unless
  the mask zeroes its position (the mask replaces it first);
* the mask is applied by replacing labels, so a nonzero mask entry at a
  position whose label already equals ``ignore_index`` still ignores it;
* the gradient is returned for every position, zero rows where ignored.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .flce_oracle import (REDUCTIONS, Forward, Problem, divisor, logit_grad, logsumexp_rows, loss_from_lse,
                          valid_positions)


@dataclasses.dataclass(frozen=True)
class CEProblem:
    ignore_index: int = -100
    reduction: str = "sum"
    num_label_tokens: int | None = None
    chunk_len: int = 32


def check_ce_problem(p: CEProblem, V: int, labels: np.ndarray) -> None:
    """Reject argument values the readings above make invalid."""
    if p.chunk_len <= 0:
        raise ValueError("chunk_len must be positive")
    if p.reduction not in REDUCTIONS:
        raise ValueError("reduction must be 'sum' or 'mean'")
    if p.num_label_tokens is not None and p.num_label_tokens <= 0:
        raise ValueError("num_label_tokens must be positive when given")
    lab = np.asarray(labels)
    bad = (lab != p.ignore_index) & ((lab < 0) | (lab >= V))
    if bad.any():
        raise ValueError("label outside [0, vocab)")


def apply_mask(labels, mask, ignore_index: int) -> np.ndarray:
    """Labels with ``ignore_index`` wherever the mask is zero."""
    lab = np.array(labels, dtype=np.int64).reshape(-1)
    if mask is None:
        return lab
    m = np.asarray(mask).reshape(-1)
    return np.where(m != 0, lab, ignore_index).astype(np.int64)


def _flat(logits, labels, mask, p: CEProblem):
    z = np.asarray(logits, dtype=np.float64)
    V = z.shape[-1]
    z = z.reshape(-1, V)
    lab = apply_mask(labels, mask, p.ignore_index)
    if lab.shape[0] != z.shape[0]:
        raise ValueError("labels must match logits.shape[:-1]")
    check_ce_problem(p, V, lab)
    return z, lab


def _as_linear_problem(p: CEProblem, V: int) -> Problem:
    return Problem(unpadded_vocab=V, softcap=0.0, ignore_index=p.ignore_index, reduction=p.reduction,
                   num_label_tokens=p.num_label_tokens)


def ce_forward(logits, labels, p: CEProblem, mask=None) -> Forward:
    """Loss, per-position losses and per-position lse (NaN where ignored)."""
    z, lab = _flat(logits, labels, mask, p)
    T, V = z.shape
    valid = valid_positions(lab, p.ignore_index)
    idx = np.nonzero(valid)[0]
    lse = np.full(T, np.nan)
    tl = np.zeros(T)
    if len(idx):
        l = logsumexp_rows(z[idx])
        lse[idx] = l
        tl[idx] = l - z[idx, lab[idx]]
    S = math.fsum(tl.tolist())
    D = divisor(_as_linear_problem(p, V), len(idx))
    loss = S / D if D != 0 else float("nan")
    return Forward(loss, tl, lse, len(idx), D, S)


def ce_backward(logits, labels, p: CEProblem, mask=None, grad_out: float = 1.0) -> np.ndarray:
    """d(grad_out * loss) / d logits, shaped [positions, vocab]."""
    z, lab = _flat(logits, labels, mask, p)
    T, V = z.shape
    valid = valid_positions(lab, p.ignore_index)
    idx = np.nonzero(valid)[0]
    out = np.zeros((T, V))
    if len(idx):
        D = divisor(_as_linear_problem(p, V), len(idx))
        out[idx] = logit_grad(z[idx], logsumexp_rows(z[idx]), lab[idx], grad_out / D)
    return out


def ce_rows(logits_rows, lab_rows, lse_rows, scale: float) -> np.ndarray:
    """Gradient rows for the given (valid) positions, from their lse."""
    z = np.asarray(logits_rows, dtype=np.float64)
    return logit_grad(z, np.asarray(lse_rows, dtype=np.float64), np.asarray(lab_rows, dtype=np.int64), scale)


def ce_lse(logits_rows) -> np.ndarray:
    """lse of the given rows (label independent)."""
    return logsumexp_rows(np.asarray(logits_rows, dtype=np.float64))


def ce_label_logits(logits_rows, lab_rows) -> np.ndarray:
    """z[i, y_i] for the given (valid) rows: the label's own logit."""
    z = np.asarray(logits_rows, dtype=np.float64)
    lab = np.asarray(lab_rows, dtype=np.int64)
    return z[np.arange(z.shape[0]), lab]


def ce_loss_from_lse(lse, label_logit, labels, p: CEProblem, vocab: int) -> Forward:
    """Per-position loss, exact total and loss from each counted position's
    lse and label logit ([T] arrays, values at ignored positions unread).
    ``labels`` are the labels after the mask was applied (:func:`apply_mask`)."""
    lab = np.asarray(labels, dtype=np.int64).reshape(-1)
    check_ce_problem(p, vocab, lab)
    return loss_from_lse(lse, label_logit, lab, _as_linear_problem(p, vocab))
