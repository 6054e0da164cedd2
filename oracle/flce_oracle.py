"""Fused linear cross-entropy: plain, slow fp64 CPU oracle.

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
constant or helper with that path.

What is computed, restated from the pages (cited by page title and section):

* "nemo_automodel.components.models.inkling2.loss",
  Inkling2FusedLinearCrossEntropy class description: bf16 hidden states are
  projected against bf16 head rows, the logit softcap and the cross-entropy
  are applied in fp32, rows at or past ``unpadded_vocab_size`` take no part in
  the softmax, and an fp32 head is first rounded to bf16.
* "nemo_automodel.components.loss.linear_ce", FusedLinearCrossEntropy.forward:
  the loss matches PyTorch's cross entropy; ``num_label_tokens`` is the global
  count that divides a sum-reduced loss; the result is a scalar.
* "nemo_automodel.components.loss.chunked_ce", _ChunkedCrossEntropySum.forward
  (``labels`` parameter): a position whose label equals ``ignore_index``
  contributes zero loss and zero gradient; compute_cross_entropy: the
  sum-reduced loss is the sum of the per-position cross-entropies.

Every step here is a plain definition evaluated in float64 on the exact
values of the bf16 inputs, so the oracle gives the mathematical value up to
float64 rounding.  The only blocking is over token rows (and, for dW rows,
over vocab rows), which bounds memory; each token's value is still computed
from its own definition.  A library matmul serves as the projection step.

Readings of points the pages leave open:

* softcap: z' = c * tanh(z / c) for c > 0; c = 0 turns it off; c < 0 is an
  error.  Its derivative is 1 - (z'/c)^2.
* reductions: 'sum' and 'mean' (PyTorch's meaning: divide by the number of
  non-ignored positions).  When ``num_label_tokens`` is given it is the
  divisor for either reduction; 0 is an error.  'none' is rejected since the
  pages' API returns a scalar.
* labels are already aligned with the hidden positions (no shift); a label
  other than ``ignore_index`` outside [0, unpadded_vocab) is an error.
* with no valid label, 'mean' without a count gives NaN (0/0) and the
  gradients are zero.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ---------------------------------------------------------------------------
# Input conversion
# ---------------------------------------------------------------------------


def round_fp32_to_bf16(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even.

    The Inkling2 loss page (class description) uses an fp32 head at its bf16
    value, the rounding sharded training applies; torch's fp32->bf16 cast
    rounds to nearest even.
    Works on the IEEE bit patterns: keep the high 16 bits after adding
    0x7FFF plus the lowest kept bit.  NaN stays NaN (quiet).  Returns the
    rounded values as float64 (exactly representable).
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(a)
    r = np.where(nan, ((u >> 16) | 0x0040) & 0xFFFF, r)
    out = (r.astype(np.uint32) << 16).view(np.float32)
    return out.astype(np.float64)


def to_f64(t) -> np.ndarray:
    """Exact float64 values of a tensor or array (bf16 / fp32 / fp64)."""
    if hasattr(t, "detach"):  # a torch tensor
        import torch

        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def head_values(W) -> np.ndarray:
    """Head weight as the float64 values of its bf16 compute copy.

    An fp32 head is rounded to bf16 (round to nearest even) first, as the
    Inkling2 loss page states; a bf16 head converts exactly.
    """
    if hasattr(W, "detach"):  # a torch tensor
        import torch

        if W.dtype == torch.float32:
            return round_fp32_to_bf16(W.detach().cpu().numpy())
        return to_f64(W)
    W = np.asarray(W)
    if W.dtype == np.float32:
        return round_fp32_to_bf16(W)
    return W.astype(np.float64)


# ---------------------------------------------------------------------------
# Problem definition
# ---------------------------------------------------------------------------

REDUCTIONS = ("sum", "mean")


@dataclasses.dataclass(frozen=True)
class Problem:
    unpadded_vocab: int
    softcap: float = 0.0
    ignore_index: int = -100
    reduction: str = "sum"
    num_label_tokens: int | None = None


def check_problem(p: Problem, T: int, H: int, V: int, labels: np.ndarray) -> None:
    """Reject the argument values the readings above make invalid."""
    if not (0 < p.unpadded_vocab <= V):
        raise ValueError("unpadded_vocab must be in (0, V]")
    if not (p.softcap >= 0.0) or math.isinf(p.softcap):
        raise ValueError("softcap must be finite and >= 0")
    if p.reduction not in REDUCTIONS:
        raise ValueError("reduction must be 'sum' or 'mean'")
    if p.num_label_tokens is not None and p.num_label_tokens <= 0:
        raise ValueError("num_label_tokens must be positive when given")
    lab = np.asarray(labels)
    bad = (lab != p.ignore_index) & ((lab < 0) | (lab >= p.unpadded_vocab))
    if bad.any():
        raise ValueError("label outside [0, unpadded_vocab)")


def valid_positions(labels, ignore_index: int) -> np.ndarray:
    """Boolean mask of positions that take part in the loss."""
    return np.asarray(labels) != ignore_index


def divisor(p: Problem, n_valid: int) -> float:
    """The normaliser D that divides the summed loss."""
    if p.num_label_tokens is not None:
        return float(p.num_label_tokens)
    if p.reduction == "mean":
        return float(n_valid)  # 0 -> NaN loss, as in PyTorch
    return 1.0


# ---------------------------------------------------------------------------
# The steps, one definition each
# ---------------------------------------------------------------------------


def project(X: np.ndarray, W: np.ndarray, Vu: int) -> np.ndarray:
    """Logits z[t, v] = sum_h X[t, h] W[v, h] for v < Vu (float64)."""
    return X @ W[:Vu].T


def softcap(z: np.ndarray, c: float) -> np.ndarray:
    """z' = c tanh(z / c) when c > 0, else z."""
    return c * np.tanh(z / c) if c > 0 else z


def softcap_slope(zp: np.ndarray, c: float):
    """d z' / d z expressed through z': 1 - (z'/c)^2 when c > 0, else 1."""
    return 1.0 - (zp / c) ** 2 if c > 0 else 1.0


def logsumexp_rows(zp: np.ndarray) -> np.ndarray:
    """log sum_v exp(z'[t, v]) per row, shifted by the row max."""
    m = zp.max(axis=1)
    return m + np.log(np.exp(zp - m[:, None]).sum(axis=1))


# ---------------------------------------------------------------------------
# Whole problem (small shapes, or token-row blocks of large ones)
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class Forward:
    loss: float            # S / D
    token_loss: np.ndarray  # [T], 0 at ignored positions
    lse: np.ndarray         # [T], NaN at ignored positions
    n_valid: int
    D: float
    S: float               # exact-summed per-token losses


def forward(X, W, labels, p: Problem, row_block: int = 1024) -> Forward:
    """Forward loss; ``X`` [T,H] and ``W`` [V,H] are float64 values."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    T, H = X.shape
    V = W.shape[0]
    check_problem(p, T, H, V, labels)
    valid = valid_positions(labels, p.ignore_index)
    idx = np.nonzero(valid)[0]
    lse = np.full(T, np.nan)
    tl = np.zeros(T)
    for b in range(0, len(idx), row_block):
        rows = idx[b:b + row_block]
        zp = softcap(project(X[rows], W, p.unpadded_vocab), p.softcap)
        l = logsumexp_rows(zp)
        lse[rows] = l
        tl[rows] = l - zp[np.arange(len(rows)), labels[rows]]
    S = math.fsum(tl.tolist())
    D = divisor(p, len(idx))
    loss = S / D if D != 0 else float("nan")
    return Forward(loss, tl, lse, len(idx), D, S)


def logit_grad(zp: np.ndarray, lse_rows: np.ndarray, lab_rows: np.ndarray, scale: float) -> np.ndarray:
    """dL/dz' for valid rows: scale * (softmax(z') - onehot(label))."""
    g = np.exp(zp - lse_rows[:, None])
    g[np.arange(len(lab_rows)), lab_rows] -= 1.0
    return scale * g


def backward(X, W, labels, p: Problem, grad_out: float = 1.0, row_block: int = 1024):
    """Gradients (dX [T,H], dW [V,H]) of grad_out * loss.

    G[t, v] = (g / D) (softmax(z')[t, v] - [v = y_t]) (1 - (z'/c)^2) for
    valid t and v < Vu, 0 elsewhere; dX = G W[:Vu]; dW[:Vu] = G^T X and the
    padding rows of dW are 0.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    T, H = X.shape
    V = W.shape[0]
    Vu = p.unpadded_vocab
    check_problem(p, T, H, V, labels)
    valid = valid_positions(labels, p.ignore_index)
    idx = np.nonzero(valid)[0]
    D = divisor(p, len(idx))
    dX = np.zeros((T, H))
    dW = np.zeros((V, H))
    if len(idx) == 0:
        return dX, dW
    scale = grad_out / D
    for b in range(0, len(idx), row_block):
        rows = idx[b:b + row_block]
        zp = softcap(project(X[rows], W, Vu), p.softcap)
        G = logit_grad(zp, logsumexp_rows(zp), labels[rows], scale) * softcap_slope(zp, p.softcap)
        dX[rows] = G @ W[:Vu]
        dW[:Vu] += G.T @ X[rows]
    return dX, dW


def dlogits(X, W, labels, p: Problem, grad_out: float = 1.0) -> np.ndarray:
    """dL/dz' as a dense [T, Vu] array (small shapes only; for invariants)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_positions(labels, p.ignore_index)
    idx = np.nonzero(valid)[0]
    D = divisor(p, len(idx))
    out = np.zeros((X.shape[0], p.unpadded_vocab))
    if len(idx):
        zp = softcap(project(X[idx], W, p.unpadded_vocab), p.softcap)
        out[idx] = logit_grad(zp, logsumexp_rows(zp), labels[idx], grad_out / D)
    return out


# ---------------------------------------------------------------------------
# Sampled evaluation for shapes too large for a dense pass
# ---------------------------------------------------------------------------


def token_lse(X_rows, W, p: Problem, row_block: int = 256) -> np.ndarray:
    """lse of the given token rows (label independent)."""
    X_rows = np.asarray(X_rows, dtype=np.float64)
    out = np.empty(X_rows.shape[0])
    for b in range(0, X_rows.shape[0], row_block):
        zp = softcap(project(X_rows[b:b + row_block], W, p.unpadded_vocab), p.softcap)
        out[b:b + row_block] = logsumexp_rows(zp)
    return out


def label_logits(X, W, labels, p: Problem) -> np.ndarray:
    """z'[t, y_t] for valid t (0 elsewhere): one dot product per token."""
    X = np.asarray(X, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_positions(labels, p.ignore_index)
    out = np.zeros(X.shape[0])
    idx = np.nonzero(valid)[0]
    z = np.einsum("th,th->t", X[idx], np.asarray(W, dtype=np.float64)[labels[idx]])
    out[idx] = softcap(z, p.softcap)
    return out


def loss_from_lse(lse, label_logit, labels, p: Problem) -> Forward:
    """The definition's last steps from each token's lse and label logit.

    For every valid position the token loss is lse_t - z'[t, y_t] (0 where
    the label is ``ignore_index``); the total S is their exact sum, and the
    loss is S / D with the normaliser of the reduction.  ``lse`` and
    ``label_logit`` are [T] arrays whose values at ignored positions are not
    read (the large workloads take them from :func:`token_lse` and
    :func:`label_logits`).
    """
    labels = np.asarray(labels, dtype=np.int64)
    valid = valid_positions(labels, p.ignore_index)
    lse = np.asarray(lse, dtype=np.float64)
    ll = np.asarray(label_logit, dtype=np.float64)
    tl = np.zeros(labels.shape[0])
    tl[valid] = lse[valid] - ll[valid]
    lse_out = np.where(valid, lse, np.nan)
    S = math.fsum(tl.tolist())
    n = int(valid.sum())
    D = divisor(p, n)
    loss = S / D if D != 0 else float("nan")
    return Forward(loss, tl, lse_out, n, D, S)


def token_rows(X, W, labels, rows, p: Problem, D: float, grad_out: float = 1.0):
    """(token loss, lse, dX rows) for the token positions ``rows``.

    Each row needs only its own logits, so this is the definition applied to
    a subset of tokens.  ``D`` is the normaliser of the whole problem.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    Vu = p.unpadded_vocab
    valid = valid_positions(labels[rows], p.ignore_index)
    tl = np.zeros(len(rows))
    lse = np.full(len(rows), np.nan)
    dX = np.zeros((len(rows), X.shape[1]))
    vr = np.nonzero(valid)[0]
    for b in range(0, len(vr), 128):
        sel = vr[b:b + 128]
        zp = softcap(project(X[rows[sel]], W, Vu), p.softcap)
        l = logsumexp_rows(zp)
        lab = labels[rows[sel]]
        lse[sel] = l
        tl[sel] = l - zp[np.arange(len(sel)), lab]
        G = logit_grad(zp, l, lab, grad_out / D) * softcap_slope(zp, p.softcap)
        dX[sel] = G @ W[:Vu]
    return tl, lse, dX


def weight_rows(X, W, labels, vrows, lse_all, p: Problem, D: float, grad_out: float = 1.0,
                token_block: int = 2048) -> np.ndarray:
    """dW rows ``vrows`` (all < Vu) summed over every valid token.

    Needs the lse of every valid token (``lse_all``, [T]), which the caller
    takes from :func:`forward` or :func:`token_lse`.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    vrows = np.asarray(vrows, dtype=np.int64)
    if np.any(vrows >= p.unpadded_vocab):
        raise ValueError("weight_rows takes usable rows only")
    idx = np.nonzero(valid_positions(labels, p.ignore_index))[0]
    out = np.zeros((len(vrows), X.shape[1]))
    Wr = W[vrows]
    scale = grad_out / D
    for b in range(0, len(idx), token_block):
        t = idx[b:b + token_block]
        zp = softcap(X[t] @ Wr.T, p.softcap)          # [tb, |R|]
        G = np.exp(zp - lse_all[t][:, None])
        G -= (labels[t][:, None] == vrows[None, :])
        G *= scale * softcap_slope(zp, p.softcap)
        out += G.T @ X[t]
    return out
