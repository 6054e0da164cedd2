"""Pins for the CPU oracle: what the pages and the mathematics fix.

Each test ties the oracle to something other than its own code: torch's
float64 cross entropy with autograd (the pages state the loss matches
PyTorch's), central finite differences, closed forms, and invariants whose
violation a dropped term, a sign error or a transposed operand would cause.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import Problem

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, T, H, V, n_ignored=0, scale=1.0):
    X = rng.standard_normal((T, H)) * scale
    W = rng.standard_normal((V, H)) * scale
    return X, W


def _labels(rng, T, Vu, n_ignored):
    y = rng.integers(0, Vu, T)
    if n_ignored:
        y[rng.permutation(T)[:n_ignored]] = -100
    return y


# ---------------------------------------------------------------------------
# bf16 rounding (Inkling2 loss page: an fp32 head is rounded to bf16)
# ---------------------------------------------------------------------------


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    vals = [rng.standard_normal(20000).astype(np.float32),
            (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormals
            np.clip(rng.standard_normal(2000) * 3e38, -3.4e38, 3.4e38).astype(np.float32)]  # near overflow
    # Exact ties: low 16 bits 0x8000 with the kept lsb both even and odd.
    hi = rng.integers(0, 0x7F7F, 4000, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    vals.append(ties)
    vals.append(-ties)
    vals.append(np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                          -np.finfo(np.float32).max, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8],
                         dtype=np.float32))
    a = np.concatenate(vals)
    ours = oracle.round_fp32_to_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    nan = oracle.round_fp32_to_bf16(np.array([np.nan], np.float32))
    assert np.isnan(nan).all()


def test_head_values_fp32_and_bf16():
    w32 = torch.randn(7, 5)
    assert np.array_equal(oracle.head_values(w32),
                          w32.to(torch.bfloat16).double().numpy())
    wb = w32.to(torch.bfloat16)
    assert np.array_equal(oracle.head_values(wb), wb.double().numpy())


# ---------------------------------------------------------------------------
# Library special case: PyTorch cross entropy in float64 with autograd
# (linear_ce page, FusedLinearCrossEntropy.forward: matches PyTorch)
# ---------------------------------------------------------------------------


def _torch_reference(X, W, y, Vu, c, reduction, n_label_tokens, grad_out):
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    z = Xt @ Wt[:Vu].T
    if c > 0:
        z = c * torch.tanh(z / c)
    yt = torch.tensor(y)
    if n_label_tokens is None:
        loss = F.cross_entropy(z, yt, ignore_index=-100, reduction=reduction)
    else:
        loss = F.cross_entropy(z, yt, ignore_index=-100, reduction="sum") / n_label_tokens
    (loss * grad_out).backward()
    return loss.item(), Xt.grad.numpy(), Wt.grad.numpy()


@pytest.mark.parametrize("c", [0.0, 30.0, 2.0])
@pytest.mark.parametrize("reduction,nlt", [("sum", None), ("mean", None), ("sum", 37), ("mean", 91)])
@pytest.mark.parametrize("Vu", [1000, 977])
def test_matches_torch_cross_entropy(c, reduction, nlt, Vu):
    rng = np.random.default_rng(hash((c, reduction, nlt, Vu)) % 2**32)
    T, H, V = 64, 128, 1000
    X = rng.standard_normal((T, H))
    W = rng.standard_normal((V, H)) * (0.02 if c == 0 else 0.5)
    y = _labels(rng, T, Vu, 6)
    g = 1.7
    p = Problem(Vu, c, -100, reduction, nlt)
    fw = oracle.forward(X, W, y, p, row_block=17)
    dX, dW = oracle.backward(X, W, y, p, grad_out=g, row_block=23)
    ref_loss, ref_dX, ref_dW = _torch_reference(X, W, y, Vu, c, reduction, nlt, g)
    assert fw.loss == pytest.approx(ref_loss, rel=1e-12, abs=1e-12)
    np.testing.assert_allclose(dX, ref_dX, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(dW, ref_dW, rtol=1e-10, atol=1e-13)
    assert np.all(dW[Vu:] == 0.0)
    # per-token losses against torch's unreduced cross entropy
    z = torch.tensor(X) @ torch.tensor(W[:Vu]).T
    if c > 0:
        z = c * torch.tanh(z / c)
    ref_tok = F.cross_entropy(z, torch.tensor(y), ignore_index=-100, reduction="none").numpy()
    np.testing.assert_allclose(fw.token_loss, ref_tok, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Central finite differences on a tiny shape (independent of the gradient
# formula: only the forward definition is used)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("c,reduction,nlt", [(2.0, "sum", None), (0.0, "mean", None), (2.0, "mean", 5)])
def test_finite_differences(c, reduction, nlt):
    rng = np.random.default_rng(11)
    T, H, V, Vu = 3, 5, 7, 6
    X = rng.standard_normal((T, H))
    W = rng.standard_normal((V, H))
    y = np.array([4, -100, 0])
    p = Problem(Vu, c, -100, reduction, nlt)
    g = 0.75
    dX, dW = oracle.backward(X, W, y, p, grad_out=g)
    eps = 1e-6

    def L(Xv, Wv):
        return g * oracle.forward(Xv, Wv, y, p).loss

    fdX = np.zeros_like(X)
    for i in range(T):
        for j in range(H):
            Xp = X.copy(); Xp[i, j] += eps
            Xm = X.copy(); Xm[i, j] -= eps
            fdX[i, j] = (L(Xp, W) - L(Xm, W)) / (2 * eps)
    fdW = np.zeros_like(W)
    for i in range(V):
        for j in range(H):
            Wp = W.copy(); Wp[i, j] += eps
            Wm = W.copy(); Wm[i, j] -= eps
            fdW[i, j] = (L(X, Wp) - L(X, Wm)) / (2 * eps)
    np.testing.assert_allclose(dX, fdX, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dW, fdW, rtol=1e-6, atol=1e-8)
    assert np.all(dX[1] == 0.0)
    assert np.all(dW[Vu:] == 0.0)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("Vu,c", [(1000, 0.0), (128256, 0.0), (256000, 30.0), (152064, 0.0), (6, 2.0)])
def test_zero_hidden_gives_log_vocab(Vu, c):
    """X = 0 makes every usable logit 0 (softcap or not): loss = log Vu per
    token, dW = 0 and dX_t = (g/D) (mean_v W[v] - W[y_t])."""
    rng = np.random.default_rng(Vu)
    T, H = 4, 8
    V = Vu + 3
    X = np.zeros((T, H))
    W = rng.standard_normal((V, H))
    y = np.array([0, Vu - 1, -100, Vu // 2])
    p = Problem(Vu, c)
    fw = oracle.forward(X, W, y, p)
    np.testing.assert_allclose(fw.token_loss[[0, 1, 3]], math.log(Vu), rtol=1e-13)
    assert fw.token_loss[2] == 0.0
    assert fw.loss == pytest.approx(3 * math.log(Vu), rel=1e-13)
    g = 2.5
    dX, dW = oracle.backward(X, W, y, p, grad_out=g)
    assert np.all(dW == 0.0)
    mean_w = W[:Vu].mean(axis=0)
    for t in (0, 1, 3):
        np.testing.assert_allclose(dX[t], g * (mean_w - W[y[t]]), rtol=1e-9, atol=1e-12)
    assert np.all(dX[2] == 0.0)


@pytest.mark.parametrize("a", [0.5, 3.0, 12.0, 40.0])
@pytest.mark.parametrize("c", [0.0, 30.0])
def test_one_hot_dominant_logit(a, c):
    """z = a e_y gives loss = log(1 + (Vu-1) exp(-a')) with a' = c tanh(a/c)
    (or a), which tends to 0 as a grows when there is no softcap."""
    Vu = 50
    W = np.eye(Vu)
    y = np.array([3, 17, 49])
    X = a * np.eye(Vu)[y]
    p = Problem(Vu, c)
    fw = oracle.forward(X, W, y, p)
    ap = c * math.tanh(a / c) if c > 0 else a
    expect = math.log1p((Vu - 1) * math.exp(-ap))
    # lse - z' cancels when the loss is small: allow fp64 cancellation.
    np.testing.assert_allclose(fw.token_loss, expect, rtol=1e-9, atol=1e-13)
    if c == 0 and a >= 40:
        assert fw.loss < 1e-14


def test_golden_closed_forms():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    env = {"e": math.e, "log": math.log, "exp": math.exp, "tanh": math.tanh}
    for case in cases:
        X = np.array(case["hidden"], dtype=np.float64)
        W = np.array(case["weight"], dtype=np.float64)
        y = np.array(case["labels"])
        p = Problem(case["unpadded_vocab"], case["softcap"], -100, case["reduction"])
        tl = np.array([eval(s, env) for s in case["token_loss"]])
        G = np.array([[eval(s, env) for s in row] for row in case["grad_logits"]])
        n_valid = int((y != -100).sum())
        D = n_valid if case["reduction"] == "mean" else 1
        fw = oracle.forward(X, W, y, p)
        np.testing.assert_allclose(fw.token_loss, tl, rtol=1e-14, atol=1e-15, err_msg=case["name"])
        assert fw.loss == pytest.approx(tl.sum() / D, rel=1e-14)
        dX, dW = oracle.backward(X, W, y, p)
        Vu = p.unpadded_vocab
        np.testing.assert_allclose(dX, (G / D) @ W[:Vu], rtol=1e-13, atol=1e-15, err_msg=case["name"])
        np.testing.assert_allclose(dW[:Vu], (G / D).T @ X, rtol=1e-13, atol=1e-15, err_msg=case["name"])
        assert np.all(dW[Vu:] == 0.0)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------


def test_softcap_bound_and_limit():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((16, 32)) * 10
    W = rng.standard_normal((40, 32)) * 10
    z = oracle.project(X, W, 40)
    for c in (0.5, 3.0, 30.0):
        assert np.all(np.abs(oracle.softcap(z, c)) <= c)
    y = rng.integers(0, 40, 16)
    W = W / 100
    a = oracle.forward(X, W, y, Problem(40, 0.0))
    b = oracle.forward(X, W, y, Problem(40, 1e7))
    assert b.loss == pytest.approx(a.loss, rel=1e-9)
    # Loss bounds: 0 <= l <= log Vu + 2c with a softcap.
    f = oracle.forward(X * 10, W * 100, y, Problem(40, 3.0))
    assert np.all(f.token_loss >= 0) and np.all(f.token_loss <= math.log(40) + 6.0 + 1e-12)


def test_gradient_rows_sum_to_zero_and_ignored_rows():
    rng = np.random.default_rng(7)
    T, H, V, Vu = 20, 16, 33, 30
    X, W = _rand_problem(rng, T, H, V)
    y = _labels(rng, T, Vu, 5)
    for c in (0.0, 4.0):
        p = Problem(Vu, c)
        G = oracle.dlogits(X, W, y, p, grad_out=1.3)
        np.testing.assert_allclose(G.sum(axis=1), 0.0, atol=1e-13)
        assert np.all(G[y == -100] == 0.0)
        dX, dW = oracle.backward(X, W, y, p, grad_out=1.3)
        assert np.all(dX[y == -100] == 0.0)
    # Without a softcap, the usable rows of dW sum to zero (each token's
    # gradient row sums to zero).
    dX, dW = oracle.backward(X, W, y, Problem(Vu, 0.0))
    np.testing.assert_allclose(dW[:Vu].sum(axis=0), 0.0, atol=1e-12)


def test_linearity_and_additivity():
    rng = np.random.default_rng(9)
    T, H, V, Vu = 24, 12, 20, 20
    X, W = _rand_problem(rng, T, H, V)
    y = _labels(rng, T, Vu, 4)
    p = Problem(Vu, 5.0)
    dX1, dW1 = oracle.backward(X, W, y, p, grad_out=1.0)
    dX3, dW3 = oracle.backward(X, W, y, p, grad_out=-3.0)
    np.testing.assert_allclose(dX3, -3.0 * dX1, rtol=1e-13)
    np.testing.assert_allclose(dW3, -3.0 * dW1, rtol=1e-13)
    # Sum reduction is additive over a partition of the tokens.
    A, B = np.arange(0, 10), np.arange(10, T)
    fa = oracle.forward(X[A], W, y[A], p)
    fb = oracle.forward(X[B], W, y[B], p)
    f = oracle.forward(X, W, y, p)
    assert f.loss == pytest.approx(fa.loss + fb.loss, rel=1e-13)
    _, dWa = oracle.backward(X[A], W, y[A], p)
    _, dWb = oracle.backward(X[B], W, y[B], p)
    np.testing.assert_allclose(dW1, dWa + dWb, rtol=1e-12, atol=1e-14)


def test_padding_rows_never_touched():
    rng = np.random.default_rng(13)
    T, H, V, Vu = 10, 8, 15, 11
    X, W = _rand_problem(rng, T, H, V)
    y = _labels(rng, T, Vu, 2)
    p = Problem(Vu, 2.0)
    Wn = W.copy()
    Wn[Vu:] = np.nan
    a = oracle.forward(X, W, y, p)
    b = oracle.forward(X, Wn, y, p)
    assert a.loss == b.loss
    dXa, dWa = oracle.backward(X, W, y, p)
    dXb, dWb = oracle.backward(X, Wn, y, p)
    assert np.array_equal(dXa, dXb) and np.array_equal(dWa, dWb)
    assert np.all(dWb[Vu:] == 0.0)
    # Same as a problem whose head has exactly the usable rows.
    c = oracle.forward(X, W[:Vu], y, p)
    assert c.loss == a.loss


def test_no_valid_tokens():
    rng = np.random.default_rng(1)
    X, W = _rand_problem(rng, 4, 6, 9)
    y = np.full(4, -100)
    s = oracle.forward(X, W, y, Problem(9, 0.0, -100, "sum"))
    assert s.loss == 0.0
    m = oracle.forward(X, W, y, Problem(9, 0.0, -100, "mean"))
    assert math.isnan(m.loss)
    dX, dW = oracle.backward(X, W, y, Problem(9, 0.0, -100, "mean"))
    assert np.all(dX == 0) and np.all(dW == 0)


def test_argument_checks():
    X = np.zeros((2, 3))
    W = np.zeros((5, 3))
    y = np.array([0, 1])
    for bad in (Problem(0), Problem(6), Problem(5, -1.0), Problem(5, float("inf")),
                Problem(5, 0.0, -100, "none"), Problem(5, 0.0, -100, "sum", 0)):
        with pytest.raises(ValueError):
            oracle.forward(X, W, y, bad)
    with pytest.raises(ValueError):
        oracle.forward(X, W, np.array([0, 5]), Problem(5))
    with pytest.raises(ValueError):
        oracle.forward(X, W, np.array([0, 4]), Problem(4))
    with pytest.raises(ValueError):
        oracle.forward(X, W, np.array([-1, 0]), Problem(5))
    # ignore_index inside the vocabulary: that class still takes part in
    # the softmax; only positions labelled with it are skipped.
    f = oracle.forward(np.ones((2, 3)), np.eye(5, 3), np.array([2, 1]), Problem(5, 0.0, 2))
    assert f.n_valid == 1 and f.token_loss[0] == 0.0


# ---------------------------------------------------------------------------
# The sampled (large-shape) entry points agree with the dense definition
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("c,reduction,nlt", [(0.0, "sum", None), (30.0, "sum", None), (0.0, "mean", 1234)])
def test_sampled_evaluation_matches_dense(c, reduction, nlt):
    rng = np.random.default_rng(21)
    T, H, V, Vu = 300, 48, 530, 512
    X = rng.standard_normal((T, H))
    W = rng.standard_normal((V, H)) / math.sqrt(H) * 3
    y = _labels(rng, T, Vu, 30)
    p = Problem(Vu, c, -100, reduction, nlt)
    fw = oracle.forward(X, W, y, p, row_block=64)
    dX, dW = oracle.backward(X, W, y, p, grad_out=0.5, row_block=64)
    rows = np.array([0, 5, 17, 63, 64, 200, 299])
    tl, lse, dXr = oracle.token_rows(X, W, y, rows, p, fw.D, grad_out=0.5)
    np.testing.assert_allclose(tl, fw.token_loss[rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dXr, dX[rows], rtol=1e-11, atol=1e-14)
    lse_all = oracle.token_lse(X, W, p, row_block=50)
    np.testing.assert_allclose(lse_all[y != -100], fw.lse[y != -100], rtol=1e-13)
    ll = oracle.label_logits(X, W, y, p)
    np.testing.assert_allclose((lse_all - ll)[y != -100], fw.token_loss[y != -100], rtol=1e-11, atol=1e-13)
    vrows = np.array([0, 1, 255, 256, 400, 511])
    dWr = oracle.weight_rows(X, W, y, vrows, lse_all, p, fw.D, grad_out=0.5, token_block=77)
    np.testing.assert_allclose(dWr, dW[vrows], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("c,reduction,nlt,Vu", [(0.0, "sum", None, 530), (30.0, "mean", None, 512),
                                                (2.0, "sum", 77, 500), (0.0, "mean", 1234, 530)])
def test_loss_from_lse_matches_torch_cross_entropy(c, reduction, nlt, Vu):
    """The sampled path of the large workloads (lse of every token, one label
    logit per token, then loss_from_lse) gives PyTorch's fp64 cross entropy:
    the per-token losses, the sum S, the divisor D and the loss."""
    rng = np.random.default_rng(31)
    T, H, V = 200, 40, 530
    X = rng.standard_normal((T, H))
    W = rng.standard_normal((V, H)) / math.sqrt(H) * 3
    y = _labels(rng, T, Vu, 23)
    p = Problem(Vu, c, -100, reduction, nlt)
    lse = oracle.token_lse(X, W, p, row_block=64)
    ll = oracle.label_logits(X, W, y, p)
    got = oracle.loss_from_lse(lse, ll, y, p)
    z = torch.tensor(X) @ torch.tensor(W[:Vu]).T
    if c > 0:
        z = c * torch.tanh(z / c)
    yt = torch.tensor(y)
    ref_tok = F.cross_entropy(z, yt, ignore_index=-100, reduction="none").numpy()
    np.testing.assert_allclose(got.token_loss, ref_tok, rtol=1e-12, atol=1e-12)
    if nlt is None:
        ref = F.cross_entropy(z, yt, ignore_index=-100, reduction=reduction).item()
    else:
        ref = F.cross_entropy(z, yt, ignore_index=-100, reduction="sum").item() / nlt
    assert got.loss == pytest.approx(ref, rel=1e-12)
    assert got.n_valid == int((y != -100).sum())
    assert got.S == pytest.approx(float(ref_tok.sum()), rel=1e-12)
    assert got.D == (nlt if nlt is not None else (got.n_valid if reduction == "mean" else 1.0))
    assert np.all(np.isnan(got.lse[y == -100]))
    # values at ignored positions are never read
    lse2 = lse.copy()
    ll2 = ll.copy()
    lse2[y == -100] = np.inf
    ll2[y == -100] = np.nan
    assert oracle.loss_from_lse(lse2, ll2, y, p).loss == got.loss
