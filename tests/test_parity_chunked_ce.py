"""GPU parity of the cross-entropy over given logits (include/chunked_ce.h)
against the CPU oracle.

Small shapes are compared element by element over every output, including
rows that are not 16-byte multiples (scalar head and tail paths) and every
mask element size.  The full-size workloads are checked on every position's
loss and lse (the oracle's lse of each row from the same logits), the total
loss, and the gradient on a seeded subset of >= 512 positions; rows of
ignored positions must be exactly zero.

Tolerances are those of the fused path: per-position loss 2e-3 absolute,
total loss 1e-4 relative, gradient rel-L2 1e-2 (a bf16 gradient carries
bf16 rounding, about 2e-3 rms).
"""
import math

import numpy as np
import pytest
import torch

import lm_head_cross_amd as L
import oracle
from tests.gpu_common import TOL_GRAD_REL_L2, TOL_TOKEN_ABS, TOL_TOTAL_REL, check_rows, rel_l2, say
from workloads import LOGIT_WORKLOADS, LogitsWorkload, make_logit_inputs, sample_logit_rows

pytestmark = pytest.mark.gpu

D = torch.device("cuda:0")


def _problem(inp):
    z = inp["logits"]
    return L.make_ce_problem(z.shape[0], z.shape[1], z.dtype, inp["ignore_index"], inp["reduction"],
                             inp["num_label_tokens"])


def _run(inp, grad_out=1.0, rows=None):
    """Forward + backward through the C ABI; CPU results."""
    z = inp["logits"].to(D)
    y = inp["labels"].to(D)
    m = None if inp.get("mask") is None else inp["mask"].to(D)
    p = _problem(inp)
    T = z.shape[0]
    loss = torch.empty((), device=D)
    lse = torch.empty(T, device=D)
    tl = torch.empty(T, device=D)
    st = torch.zeros((), dtype=torch.int32, device=D)
    L.chunked_ce_forward(p, z, y, loss, lse, mask=m, token_loss=tl, device_status=st)
    g = torch.tensor(grad_out, device=D)
    dz = torch.empty_like(z)
    L.chunked_ce_backward(p, z, y, lse, g, dz, mask=m, device_status=st)
    torch.cuda.synchronize()
    out = {"loss": loss.item(), "lse": lse.cpu(), "token_loss": tl.cpu(), "status": st.item()}
    if rows is None:
        out["dz"] = dz.float().cpu()
    else:
        out["dz_rows"] = dz[torch.from_numpy(rows).to(D)].float().cpu()
        out["dz_dev"] = dz
    return out


def _ref_problem(inp):
    return oracle.CEProblem(ignore_index=inp["ignore_index"], reduction=inp["reduction"],
                            num_label_tokens=inp["num_label_tokens"])


def _check_full(inp, res, grad_out=1.0, label=""):
    z = oracle.to_f64(inp["logits"].cpu())
    y = inp["labels"].cpu().numpy()
    m = None if inp.get("mask") is None else inp["mask"].cpu().numpy()
    p = _ref_problem(inp)
    ref = oracle.ce_forward(z, y, p, mask=m)
    counted = ~np.isnan(ref.lse)
    tl_err = np.abs(res["token_loss"].double().numpy() - ref.token_loss).max()
    lse_err = np.abs(res["lse"].double().numpy()[counted] - ref.lse[counted]).max() if counted.any() else 0.0
    say(f"  {label}: loss gpu={res['loss']:.9g} ref={ref.loss:.9g}  max|dl|={tl_err:.3g} max|dlse|={lse_err:.3g}")
    assert tl_err <= TOL_TOKEN_ABS and lse_err <= TOL_TOKEN_ABS
    assert np.all(res["lse"].numpy()[~counted] == 0)
    if math.isnan(ref.loss):
        assert math.isnan(res["loss"])
    else:
        assert abs(res["loss"] - ref.loss) <= TOL_TOTAL_REL * max(abs(ref.loss), 1e-30)
    gref = oracle.ce_backward(z, y, p, mask=m, grad_out=grad_out)
    e = rel_l2(res["dz"].double().numpy(), gref)
    say(f"  {label}: grad rel-L2 {e:.3g}")
    assert e <= TOL_GRAD_REL_L2
    check_rows(res["dz"].double().numpy()[counted], gref[counted], label)
    assert torch.all(res["dz"][torch.from_numpy(~counted)] == 0)


def _small(key, **kw):
    base = dict(name=key, std=2.0)
    base.update(kw)
    return LogitsWorkload(key=key, **base)


SMALL = {
    "ce1_fp32_unaligned_rows": LOGIT_WORKLOADS["ce1"],
    "bf16_odd_vocab": _small("ce101", T=300, V=4099, dtype="bf16", ignore_frac=0.05),
    "fp32_masked_mean_count": _small("ce102", T=257, V=3001, dtype="fp32", ignore_frac=0.2, reduction="mean",
                                     normalise_by_count=True, use_mask=True),
    "bf16_runs_mean_peaked": _small("ce103", T=2000, V=2048, dtype="bf16", std=3.0, ignore="runs",
                                    reduction="mean", peak=12.0),
    "bf16_one_column_short_rows": _small("ce104", T=100, V=7, dtype="bf16", ignore_frac=0.1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    w = SMALL[name]
    say(f"case {name}: T={w.T} V={w.V} {w.dtype} {w.reduction}")
    inp = make_logit_inputs(w)
    res = _run(inp)
    assert res["status"] == 0
    _check_full(inp, res, label=name)


def test_grad_out_scaling():
    inp = make_logit_inputs(SMALL["fp32_masked_mean_count"])
    _check_full(inp, _run(inp, grad_out=-2.5), grad_out=-2.5, label="grad_out=-2.5")


@pytest.mark.parametrize("mdtype", [torch.bool, torch.uint8, torch.int8, torch.int16, torch.int32, torch.int64,
                                    torch.float32])
def test_mask_element_types(mdtype):
    inp = make_logit_inputs(SMALL["fp32_masked_mean_count"])
    inp = dict(inp)
    inp["mask"] = (inp["mask"] != 0).to(mdtype) * (3 if mdtype not in (torch.bool,) else 1)
    if mdtype == torch.bool:
        inp["mask"] = inp["mask"].bool()
    _check_full(inp, _run(inp), label=f"mask {mdtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_negative_infinite_columns(dtype):
    """Logits at -inf (masked vocabulary entries): a span of columns long
    enough that whole 16-byte vectors, and lanes' first vectors, hold only
    -inf, plus scattered single columns and the row's last column.  They add
    nothing to the softmax and get a zero gradient; every result stays
    finite and matches the oracle."""
    key = "ce105" if dtype == "bf16" else "ce106"
    inp = dict(make_logit_inputs(_small(key, T=64, V=4099, dtype=dtype, ignore_frac=0.1)))
    z = inp["logits"].clone()
    T, V = z.shape
    dead = np.concatenate([np.arange(8, 3000), np.arange(3100, 4099, 37), [V - 1]])
    z[:, torch.from_numpy(dead)] = float("-inf")
    z[5, :] = float("-inf")
    z[5, 3001] = 1.5
    inp["logits"] = z
    y = inp["labels"].clone()
    live = np.setdiff1d(np.arange(V), dead)
    bad = np.isin(y.numpy(), dead)
    y[torch.from_numpy(bad)] = torch.from_numpy(live[np.arange(int(bad.sum())) % len(live)])
    y[5] = 3001
    inp["labels"] = y
    res = _run(inp)
    assert res["status"] == 0
    assert math.isfinite(res["loss"]) and torch.all(torch.isfinite(res["lse"]))
    assert torch.all(torch.isfinite(res["dz"]))
    assert torch.all(res["dz"][:, torch.from_numpy(dead)] == 0)
    _check_full(inp, res, label=f"-inf columns {dtype}")


def test_deterministic_repeat():
    inp = make_logit_inputs(SMALL["bf16_runs_mean_peaked"])
    a, b = _run(inp), _run(inp)
    assert a["loss"] == b["loss"]
    for k in ("lse", "token_loss", "dz"):
        assert torch.equal(a[k], b[k]), k


def test_ignored_rows_never_read():
    """NaN in the rows of ignored positions changes nothing."""
    inp = make_logit_inputs(SMALL["bf16_odd_vocab"])
    a = _run(inp)
    poisoned = dict(inp)
    z = inp["logits"].clone()
    z[inp["labels"] == -100] = float("nan")
    poisoned["logits"] = z
    b = _run(poisoned)
    assert a["loss"] == b["loss"]
    for k in ("lse", "token_loss", "dz"):
        assert torch.equal(a[k], b[k]), k


def test_bad_labels_flagged_and_skipped():
    inp = make_logit_inputs(SMALL["bf16_odd_vocab"])
    y = inp["labels"].clone()
    bad = dict(inp)
    yb = y.clone()
    yb[[1, 7]] = torch.tensor([5000, -5])
    bad["labels"] = yb
    res = _run(bad)
    assert res["status"] == 1
    ref = dict(inp)
    yr = y.clone()
    yr[[1, 7]] = -100
    ref["labels"] = yr
    _check_full(ref, res, label="bad labels as ignored")


@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_all_positions_ignored(reduction):
    inp = dict(make_logit_inputs("ce1"))
    inp["labels"] = torch.full_like(inp["labels"], -100)
    inp["reduction"] = reduction
    res = _run(inp)
    assert (res["loss"] == 0.0) if reduction == "sum" else math.isnan(res["loss"])
    assert torch.all(res["dz"] == 0) and torch.all(res["lse"] == 0)


def test_empty_batch():
    p = L.make_ce_problem(0, 100, torch.float32, reduction="mean")
    z = torch.empty((0, 100), device=D)
    y = torch.empty(0, dtype=torch.int64, device=D)
    loss = torch.zeros((), device=D)
    L.chunked_ce_forward(p, z, y, loss, torch.empty(0, device=D))
    L.chunked_ce_backward(p, z, y, torch.empty(0, device=D), torch.ones((), device=D), torch.empty_like(z))
    torch.cuda.synchronize()
    assert math.isnan(loss.item())


def test_module_mask_rewrites_labels_and_autograd():
    """ChunkedCrossEntropy.forward with a mask: the masked positions' labels
    become ignore_index in the caller's tensor (the page's documented side
    effect), and loss.backward() gives the oracle's gradient."""
    inp = make_logit_inputs(SMALL["fp32_masked_mean_count"])
    T, V = inp["logits"].shape
    z = inp["logits"].to(D).reshape(1, T, V).clone().requires_grad_(True)
    y = inp["labels"].to(D).reshape(1, T).clone()
    m = inp["mask"].to(D).reshape(1, T)
    mod = L.ChunkedCrossEntropy(chunk_len=16, reduction="mean")
    loss = mod(z, y, mask=m, num_label_tokens=inp["num_label_tokens"])
    loss.backward()
    torch.cuda.synchronize()
    y_ref = np.where(inp["mask"].numpy() != 0, inp["labels"].numpy(), -100)
    assert np.array_equal(y.cpu().numpy().reshape(-1), y_ref)
    zc = oracle.to_f64(inp["logits"])
    p = oracle.CEProblem(reduction="mean", num_label_tokens=inp["num_label_tokens"])
    ref = oracle.ce_forward(zc, y_ref, p)
    assert abs(loss.item() - ref.loss) <= TOL_TOTAL_REL * abs(ref.loss)
    e = rel_l2(z.grad.reshape(T, V).double().cpu().numpy(), oracle.ce_backward(zc, y_ref, p))
    assert e <= TOL_GRAD_REL_L2
    # compute_cross_entropy is the same sum-reduced loss
    s = L.compute_cross_entropy(inp["logits"].to(D), torch.from_numpy(y_ref).to(D))
    assert abs(s.item() - oracle.ce_forward(zc, y_ref, oracle.CEProblem()).loss) <= TOL_TOTAL_REL * abs(s.item())


# ---------------------------------------------------------------------------
# Full-size workloads, sampled gradient checks
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("key", ["ce2", "ce3", "ce4"])
def test_workload_full_size(key):
    w = LOGIT_WORKLOADS[key]
    say(f"workload {key}: {w.name}")
    inp = make_logit_inputs(w, device="cuda:0")
    y = inp["labels"].cpu().numpy()
    m = None if inp["mask"] is None else inp["mask"].cpu().numpy()
    yeff = oracle.apply_mask(y, m, -100)
    counted = yeff != -100
    rows = sample_logit_rows(w, counted)
    res = _run(inp, rows=rows)
    assert res["status"] == 0
    assert torch.all(res["dz_dev"][torch.from_numpy(~counted).to(D)] == 0)
    del res["dz_dev"]
    # every position's lse from the same logits, in row blocks
    zc = inp["logits"].cpu()
    lse_ref = np.full(w.T, np.nan)
    idx = np.nonzero(counted)[0]
    for b in range(0, len(idx), 512):
        r = idx[b:b + 512]
        lse_ref[r] = oracle.ce_lse(oracle.to_f64(zc[torch.from_numpy(r)]))
    ll_ref = np.zeros(w.T)
    for b in range(0, len(idx), 512):
        r = idx[b:b + 512]
        ll_ref[r] = oracle.ce_label_logits(oracle.to_f64(zc[torch.from_numpy(r)]), yeff[r])
    ref = oracle.ce_loss_from_lse(lse_ref, ll_ref, yeff, _ref_problem(inp), w.V)
    tl_ref, ref_loss, D_ = ref.token_loss, ref.loss, ref.D
    tl_err = np.abs(res["token_loss"].double().numpy() - tl_ref).max()
    lse_err = np.abs(res["lse"].double().numpy()[counted] - lse_ref[counted]).max()
    say(f"  loss gpu={res['loss']:.9g} ref={ref_loss:.9g} max|dl|={tl_err:.3g} max|dlse|={lse_err:.3g}")
    assert tl_err <= TOL_TOKEN_ABS and lse_err <= TOL_TOKEN_ABS
    assert abs(res["loss"] - ref_loss) <= TOL_TOTAL_REL * abs(ref_loss)
    # gradient rows
    rc = rows[counted[rows]]
    sel = np.isin(rows, rc)
    g_ref = oracle.ce_rows(oracle.to_f64(zc[torch.from_numpy(rc)]), yeff[rc], lse_ref[rc], 1.0 / D_)
    e = rel_l2(res["dz_rows"][torch.from_numpy(sel)].double().numpy(), g_ref)
    say(f"  grad rel-L2 over {len(rc)} counted rows = {e:.3g}")
    assert e <= TOL_GRAD_REL_L2
    check_rows(res["dz_rows"][torch.from_numpy(sel)].double().numpy(), g_ref, "d_logits")
    assert torch.all(res["dz_rows"][torch.from_numpy(~sel)] == 0)


def test_one_class():
    """V = 1: the softmax over one class is 1, so every counted position's
    loss and gradient are exactly 0; the kernels reach them up to rounding."""
    g = torch.Generator().manual_seed(3)
    for dtype in (torch.bfloat16, torch.float32):
        z = (torch.randn(300, 1, generator=g) * 5).to(dtype)
        y = torch.zeros(300, dtype=torch.int64)
        y[::7] = -100
        inp = {"logits": z, "labels": y, "mask": None, "ignore_index": -100, "reduction": "sum",
               "num_label_tokens": None}
        ref = oracle.ce_forward(oracle.to_f64(z), y.numpy(), _ref_problem(inp))
        assert ref.loss == 0.0
        res = _run(inp)
        assert res["status"] == 0
        assert res["token_loss"].abs().max().item() <= 1e-5
        assert res["dz"].abs().max().item() <= 1e-6
        counted = y != -100
        zc = z[counted, 0].float()
        assert torch.all((res["lse"][counted] - zc).abs() <= 1e-6 * (1 + zc.abs()))


def _sweep_case(i):
    rng = np.random.default_rng(9000 + i)
    T = int(rng.choice([1, 2, 63, 64, 65, 255, 257] + [int(x) for x in rng.integers(1, 3001, 3)]))
    V = int(rng.choice([1, 2, 3, 7, 8, 9, 15, 16, 17] + [int(x) for x in rng.integers(2, 20001, 5)]))
    ignore_frac = float(rng.choice([0.0, 0.05, 0.5])) if T >= 20 else 0.0
    return _small(f"ce{200 + i}", T=T, V=V, dtype=str(rng.choice(["bf16", "fp32"])),
                  std=float(rng.choice([0.5, 2.0, 5.0])), ignore_frac=ignore_frac,
                  reduction=str(rng.choice(["sum", "mean"])), use_mask=bool(rng.random() < 0.3),
                  peak=float(rng.choice([0.0, 0.0, 10.0])))


@pytest.mark.parametrize("i", range(32))
def test_random_small_problem(i):
    """A seeded sweep of random small problems (row lengths of every
    alignment, so the scalar head and tail paths vary; bf16 and fp32; masks;
    peaked labels) against the oracle, element by element."""
    w = _sweep_case(i)
    say(f"sweep {i}: T={w.T} V={w.V} {w.dtype} std={w.std} {w.reduction} ignore={w.ignore_frac} "
        f"mask={w.use_mask} peak={w.peak}")
    inp = make_logit_inputs(w)
    res = _run(inp)
    assert res["status"] == 0
    _check_full(inp, res, label=f"sweep{i}")
