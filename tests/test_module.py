"""The autograd modules (FusedLinearCrossEntropy, Inkling2FusedLinearCrossEntropy).

CPU: constructor and argument checks, which fail before any device call.
GPU: loss.backward() through the modules against the oracle, with batched
[B, S, H] hidden states, an unpadded vocabulary, a count divisor, a scaled
upstream gradient, and bf16 / fp32 heads.
"""
import numpy as np
import pytest
import torch

import lm_head_cross_amd as L


def test_constructor_checks():
    with pytest.raises(ValueError):
        L.FusedLinearCrossEntropy(reduction="none")
    with pytest.raises(ValueError):
        L.FusedLinearCrossEntropy(logit_softcapping=-1.0)
    with pytest.raises(ValueError):
        L.FusedLinearCrossEntropy(unpadded_vocab_size=0)
    with pytest.raises(ValueError):
        L.Inkling2FusedLinearCrossEntropy(unpadded_vocab_size=None)
    m = L.Inkling2FusedLinearCrossEntropy(1000)
    assert (m.unpadded_vocab_size, m.logit_softcapping, m.ignore_index, m.reduction) == (1000, 30.0, -100, "sum")
    m = L.FusedLinearCrossEntropy()
    assert (m.unpadded_vocab_size, m.logit_softcapping, m.ignore_index, m.reduction) == (None, 0, -100, "sum")


def test_sharded_head_and_group_refused_on_one_gpu():
    m = L.FusedLinearCrossEntropy()
    h = torch.zeros(4, 128, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    w = torch.zeros(16, 128, dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError):
        m(h, y, w, grad_reduce_group=object())


def test_input_dtype_and_shape_checks():
    f = L.fused_linear_cross_entropy
    w = torch.zeros(16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        f(torch.zeros(4, 128, dtype=torch.float32), torch.zeros(4, dtype=torch.int64), w)
    with pytest.raises(ValueError):
        f(torch.zeros(4, 128, dtype=torch.bfloat16), torch.zeros(5, dtype=torch.int64), w)
    with pytest.raises(ValueError):
        f(torch.zeros(4, 128, dtype=torch.bfloat16), torch.zeros(4, dtype=torch.int64), w.half())


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------


def _inputs(seed, B, S, H, V, vu, ignore_frac, head_dtype):
    g = torch.Generator().manual_seed(seed)
    X = (torch.randn(B, S, H, generator=g)).to(torch.bfloat16)
    W = (torch.randn(V, H, generator=g) * 0.08).to(head_dtype)
    y = torch.randint(0, vu, (B, S), generator=g)
    ign = torch.rand(B, S, generator=g) < ignore_frac
    y[ign] = -100
    return X, W, y


def _oracle(X, W, y, vu, softcap, reduction, count, grad_out):
    import oracle

    H = X.shape[-1]
    Xo = oracle.to_f64(X.reshape(-1, H))
    Wo = oracle.head_values(W)
    yo = y.reshape(-1).numpy()
    p = oracle.Problem(vu, softcap, -100, reduction, count)
    fw = oracle.forward(Xo, Wo, yo, p)
    dX, dW = oracle.backward(Xo, Wo, yo, p, grad_out=grad_out)
    return fw.loss, dX.reshape(X.shape), dW


def _rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


CASES = {
    # name: (module factory, B, S, H, V, unpadded, softcap, reduction, count, head dtype, grad_out)
    "mean_fp32_head": (lambda: L.FusedLinearCrossEntropy(reduction="mean", unpadded_vocab_size=1050),
                       2, 300, 256, 1100, 1050, 0.0, "mean", None, torch.float32, 1.5),
    "sum_bf16_head_count": (lambda: L.FusedLinearCrossEntropy(), 3, 170, 384, 1300, 1300, 0.0, "sum", 400,
                            torch.bfloat16, -0.75),
    "inkling2_softcap": (lambda: L.Inkling2FusedLinearCrossEntropy(2000), 1, 513, 128, 2048, 2000, 30.0, "sum",
                         None, torch.float32, 1.0),
}


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_module_backward_matches_oracle(name):
    make, B, S, H, V, vu, c, red, count, hdt, g = CASES[name]
    print(f"module case {name}: B={B} S={S} H={H} V={V} Vu={vu} c={c} {red} count={count} head={hdt}", flush=True)
    X, W, y = _inputs(11 + list(CASES).index(name), B, S, H, V, vu, 0.1, hdt)
    d = torch.device("cuda:0")
    Xd = X.to(d).requires_grad_(True)
    Wd = W.to(d).requires_grad_(True)
    loss = make()(Xd, y.to(d), Wd, num_label_tokens=count)
    assert loss.shape == () and loss.dtype == torch.float32
    (loss * g).backward()
    torch.cuda.synchronize()
    ref_loss, ref_dX, ref_dW = _oracle(X, W, y, vu, c, red, count, g)
    assert abs(loss.item() - ref_loss) <= 1e-4 * abs(ref_loss) + 1e-6, (loss.item(), ref_loss)
    assert Xd.grad.dtype == torch.bfloat16 and Xd.grad.shape == X.shape
    assert Wd.grad.dtype == hdt and Wd.grad.shape == W.shape
    assert _rel_l2(Xd.grad.double().cpu().numpy(), ref_dX) <= 1e-2
    assert _rel_l2(Wd.grad.double().cpu().numpy(), ref_dW) <= 1e-2
    ignored = (y == -100).to(d)
    assert torch.all(Xd.grad[ignored] == 0)
    assert torch.all(Wd.grad[vu:] == 0)


@pytest.mark.gpu
def test_module_rejects_label_outside_usable_vocabulary():
    """A label in [Vu, V) or negative (not ignore_index) raises ValueError by
    default, as PyTorch's cross entropy does; with check_labels off the
    position is skipped like an ignored one (the oracle's loss without it)."""
    import oracle

    d = torch.device("cuda:0")
    X, W, y = _inputs(5, 1, 200, 128, 1100, 1000, 0.1, torch.bfloat16)
    for bad_label in (1000, 1099, -3):
        yb = y.clone()
        yb[0, 17] = bad_label
        with pytest.raises(ValueError):
            L.FusedLinearCrossEntropy(unpadded_vocab_size=1000)(X.to(d), yb.to(d), W.to(d))
        with pytest.raises(ValueError):
            L.Inkling2FusedLinearCrossEntropy(1000)(X.to(d), yb.to(d), W.to(d))
    yb = y.clone()
    yb[0, 17] = 1050
    loss = L.FusedLinearCrossEntropy(unpadded_vocab_size=1000, check_labels=False)(X.to(d), yb.to(d), W.to(d))
    yr = y.clone()
    yr[0, 17] = -100
    ref = oracle.forward(oracle.to_f64(X.reshape(-1, 128)), oracle.head_values(W), yr.reshape(-1).numpy(),
                         oracle.Problem(1000))
    assert abs(loss.item() - ref.loss) <= 1e-4 * abs(ref.loss)


@pytest.mark.gpu
def test_chunked_module_rejects_label_outside_vocabulary():
    d = torch.device("cuda:0")
    g = torch.Generator().manual_seed(9)
    z = torch.randn(50, 300, generator=g).to(d)
    y = torch.randint(0, 300, (50,), generator=g).to(d)
    y[3] = 300
    with pytest.raises(ValueError):
        L.ChunkedCrossEntropy()(z, y)
    with pytest.raises(ValueError):
        L.compute_cross_entropy(z, y)
    loss = L.ChunkedCrossEntropy(check_labels=False)(z, y)
    yr = y.clone()
    yr[3] = -100
    assert abs(loss.item() - L.compute_cross_entropy(z, yr).item()) <= 1e-5 * abs(loss.item())
