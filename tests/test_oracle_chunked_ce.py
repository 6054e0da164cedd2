"""Pins of the cross-entropy-over-logits oracle (the chunked CE page).

Each test checks the oracle against something other than itself: closed
forms, PyTorch's own fp64 cross entropy on the CPU (the page says the loss
matches it), finite differences, and the fused linear oracle on logits
X W^T.  A plausible slip in the oracle (a dropped normaliser, a wrong sign,
a mask applied the wrong way round, a transposed index) fails one of them.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import CEProblem, ce_backward, ce_forward

RNG = np.random.default_rng(7)


def _case(T=9, V=13, scale=2.0, ignore=(2, 5)):
    z = RNG.normal(0.0, scale, (T, V))
    y = RNG.integers(0, V, T)
    y[list(ignore)] = -100
    return z, y


def test_uniform_logits_give_log_vocab():
    # Uniform logits: every position's loss is log V exactly.
    z = np.full((5, 1000), 3.25)
    y = np.array([0, 999, 17, -100, 500])
    f = ce_forward(z, y, CEProblem())
    np.testing.assert_allclose(f.token_loss[[0, 1, 2, 4]], math.log(1000), rtol=1e-14)
    assert f.token_loss[3] == 0.0
    assert f.loss == pytest.approx(4 * math.log(1000), rel=1e-14)


def test_one_hot_dominant_closed_form():
    # z_y = a, others 0: loss = log(1 + (V-1) e^{-a}).
    V = 50
    for a in (0.0, 1.5, 10.0, 40.0):
        z = np.zeros((1, V))
        z[0, 7] = a
        f = ce_forward(z, np.array([7]), CEProblem())
        # lse - z_y cancels to within a few ulp of the lse (about a)
        assert f.loss == pytest.approx(math.log1p((V - 1) * math.exp(-a)), rel=1e-12, abs=4 * np.spacing(a + 1.0))


@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_matches_torch_cross_entropy_fp64(reduction):
    z, y = _case()
    f = ce_forward(z, y, CEProblem(reduction=reduction))
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    ref = F.cross_entropy(zt, torch.tensor(y), ignore_index=-100, reduction=reduction)
    assert f.loss == pytest.approx(ref.item(), rel=1e-13)
    ref.backward()
    np.testing.assert_allclose(ce_backward(z, y, CEProblem(reduction=reduction)), zt.grad.numpy(), rtol=1e-12,
                               atol=1e-15)


def test_num_label_tokens_divides_either_reduction():
    z, y = _case()
    s = ce_forward(z, y, CEProblem()).S
    for red in ("sum", "mean"):
        f = ce_forward(z, y, CEProblem(reduction=red, num_label_tokens=11))
        assert f.loss == pytest.approx(s / 11, rel=1e-14)
        g = ce_backward(z, y, CEProblem(reduction=red, num_label_tokens=11))
        np.testing.assert_allclose(g, ce_backward(z, y, CEProblem()) / 11, rtol=1e-13, atol=1e-16)


def test_mask_is_label_replacement():
    z, y = _case(ignore=())
    mask = np.ones(len(y), dtype=np.int64)
    mask[[1, 4]] = 0
    mask[6] = -3  # any nonzero entry counts
    y_bad = y.copy()
    y_bad[4] = 10 ** 6  # masked out: replaced before the range check
    f = ce_forward(z, y_bad, CEProblem(), mask=mask)
    y_ref = y.copy()
    y_ref[[1, 4]] = -100
    ref = ce_forward(z, y_ref, CEProblem())
    assert f.loss == ref.loss and f.n_valid == len(y) - 2
    np.testing.assert_array_equal(ce_backward(z, y_bad, CEProblem(), mask=mask), ce_backward(z, y_ref, CEProblem()))
    # torch with the replaced labels
    zt = torch.tensor(z)
    assert f.loss == pytest.approx(F.cross_entropy(zt, torch.tensor(y_ref), reduction="sum").item(), rel=1e-13)
    np.testing.assert_array_equal(oracle.apply_mask(y, mask, -7), np.where(mask != 0, y, -7))


def test_finite_differences():
    z, y = _case(T=3, V=7, ignore=(1,))
    p = CEProblem(reduction="mean")
    g = ce_backward(z, y, p, grad_out=1.7)
    eps = 1e-6
    num = np.zeros_like(z)
    for i in range(z.shape[0]):
        for j in range(z.shape[1]):
            zp, zm = z.copy(), z.copy()
            zp[i, j] += eps
            zm[i, j] -= eps
            num[i, j] = 1.7 * (ce_forward(zp, y, p).loss - ce_forward(zm, y, p).loss) / (2 * eps)
    np.testing.assert_allclose(g, num, rtol=1e-7, atol=1e-9)


def test_gradient_invariants():
    z, y = _case()
    g = ce_backward(z, y, CEProblem(), grad_out=2.5)
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-13)  # rows sum to zero
    assert np.all(g[y == -100] == 0)                            # ignored rows are exactly zero
    np.testing.assert_allclose(g, 2.5 * ce_backward(z, y, CEProblem()), rtol=1e-14)  # linear in grad_out
    # the label entry is the only negative one
    rows = np.nonzero(y != -100)[0]
    assert np.all(g[rows, y[rows]] < 0)
    off = g[rows].copy()
    off[np.arange(len(rows)), y[rows]] = 0
    assert np.all(off >= 0)


def test_shift_invariance_with_large_logits():
    # Adding a constant to a row changes neither its loss nor its gradient
    # (the lse is taken relative to the row max).
    z, y = _case()
    shift = RNG.normal(0, 1e4, (z.shape[0], 1))
    a, b = ce_forward(z, y, CEProblem()), ce_forward(z + shift, y, CEProblem())
    np.testing.assert_allclose(a.token_loss, b.token_loss, atol=1e-8)
    np.testing.assert_allclose(ce_backward(z, y, CEProblem()), ce_backward(z + shift, y, CEProblem()), atol=1e-12)


def test_agrees_with_fused_linear_oracle():
    # Logits given as X W^T equal the fused linear loss with no softcap and
    # no padding, and their gradient is the fused path's dL/dz'.
    X = RNG.normal(0, 1, (11, 6))
    W = RNG.normal(0, 0.7, (17, 6))
    y = RNG.integers(0, 17, 11)
    y[[0, 8]] = -100
    lp = oracle.Problem(unpadded_vocab=17, reduction="mean")
    a = oracle.forward(X, W, y, lp)
    b = ce_forward(X @ W.T, y, CEProblem(reduction="mean"))
    assert b.loss == pytest.approx(a.loss, rel=1e-13)
    np.testing.assert_allclose(b.lse[y != -100], a.lse[y != -100], rtol=1e-14)
    np.testing.assert_allclose(ce_backward(X @ W.T, y, CEProblem(reduction="mean")), oracle.dlogits(X, W, y, lp),
                               rtol=1e-12, atol=1e-16)


def test_leading_dimensions_flatten():
    z, y = _case(T=12)
    f = ce_forward(z.reshape(3, 4, -1), y.reshape(3, 4), CEProblem())
    assert f.loss == ce_forward(z, y, CEProblem()).loss


def test_validation():
    z, y = _case()
    with pytest.raises(ValueError):
        ce_forward(z, y, CEProblem(chunk_len=0))
    with pytest.raises(ValueError):
        ce_forward(z, y, CEProblem(reduction="none"))
    with pytest.raises(ValueError):
        ce_forward(z, y, CEProblem(num_label_tokens=0))
    bad = y.copy()
    bad[0] = z.shape[1]
    with pytest.raises(ValueError):
        ce_forward(z, bad, CEProblem())


def test_no_valid_position():
    z, _ = _case()
    y = np.full(z.shape[0], -100)
    assert ce_forward(z, y, CEProblem()).loss == 0.0
    assert math.isnan(ce_forward(z, y, CEProblem(reduction="mean")).loss)
    assert np.all(ce_backward(z, y, CEProblem(reduction="mean")) == 0)


@pytest.mark.parametrize("reduction,nlt,g", [("sum", None, 1.0), ("mean", None, -0.75), ("sum", 40, 2.5)])
def test_row_helpers_match_whole_problem(reduction, nlt, g):
    """ce_lse, ce_label_logits, ce_rows and ce_loss_from_lse (the sampled path
    of the full-size logits workloads) give, row by row, what ce_forward and
    ce_backward give for the whole problem, and PyTorch's fp64 cross entropy.
    Logit scales differ by row, so swapping ce_rows' lse and label arguments,
    or taking another row's lse, fails."""
    rng = np.random.default_rng(13)
    T, V = 40, 97
    z = rng.normal(0.0, 1.0, (T, V)) * rng.uniform(0.5, 6.0, (T, 1)) + rng.normal(0.0, 5.0, (T, 1))
    y = rng.integers(0, V, T)
    y[[3, 11, 30]] = -100
    p = CEProblem(reduction=reduction, num_label_tokens=nlt)
    fw = ce_forward(z, y, p)
    dz = ce_backward(z, y, p, grad_out=g)
    idx = np.nonzero(y != -100)[0]
    lse_rows = oracle.ce_lse(z[idx])
    np.testing.assert_allclose(lse_rows, fw.lse[idx], rtol=1e-14)
    np.testing.assert_allclose(lse_rows, torch.logsumexp(torch.tensor(z[idx]), dim=1).numpy(), rtol=1e-13)
    ll = oracle.ce_label_logits(z[idx], y[idx])
    assert np.array_equal(ll, z[idx, y[idx]])
    lse_all = np.full(T, np.nan)
    lse_all[idx] = lse_rows
    ll_all = np.zeros(T)
    ll_all[idx] = ll
    got = oracle.ce_loss_from_lse(lse_all, ll_all, y, p, V)
    np.testing.assert_allclose(got.token_loss, fw.token_loss, rtol=1e-13, atol=1e-14)
    assert got.loss == pytest.approx(fw.loss, rel=1e-13)
    assert (got.S, got.D, got.n_valid) == pytest.approx((fw.S, fw.D, fw.n_valid), rel=1e-13)
    zt = torch.tensor(z, requires_grad=True)
    red = "sum" if nlt is not None else reduction
    ref = F.cross_entropy(zt, torch.tensor(y), ignore_index=-100, reduction=red)
    if nlt is not None:
        ref = ref / nlt
    (ref * g).backward()
    assert got.loss == pytest.approx(ref.item(), rel=1e-12)
    rows = oracle.ce_rows(z[idx], y[idx], lse_rows, g / fw.D)
    np.testing.assert_allclose(rows, dz[idx], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(rows, zt.grad.numpy()[idx], rtol=1e-11, atol=1e-15)


def test_negative_infinite_logits():
    """Columns at -inf (masked vocabulary entries) add nothing to the softmax:
    the loss and the other columns' gradient equal those of the problem
    without the columns, PyTorch agrees, and the gradient there is 0."""
    rng = np.random.default_rng(17)
    T, V = 12, 40
    z = rng.normal(0.0, 3.0, (T, V))
    dead = np.array([0, 1, 2, 9, 20, 21, 39])
    z[:, dead] = -np.inf
    keep = np.setdiff1d(np.arange(V), dead)
    y = keep[rng.integers(0, len(keep), T)]
    y[4] = -100
    p = CEProblem(reduction="mean")
    fw = ce_forward(z, y, p)
    dz = ce_backward(z, y, p)
    remap = np.full(V, -1)
    remap[keep] = np.arange(len(keep))
    y_k = np.where(y == -100, -100, remap[np.maximum(y, 0)])
    ref = ce_forward(z[:, keep], y_k, p)
    assert np.isfinite(fw.loss) and fw.loss == pytest.approx(ref.loss, rel=1e-14)
    np.testing.assert_allclose(dz[:, keep], ce_backward(z[:, keep], y_k, p), rtol=1e-14, atol=1e-17)
    assert np.all(dz[:, dead] == 0.0)
    zt = torch.tensor(z)
    assert fw.loss == pytest.approx(F.cross_entropy(zt, torch.tensor(y), ignore_index=-100).item(), rel=1e-13)
