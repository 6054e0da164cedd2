"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small shapes are compared element by element over every output; they span
several 256-wide tiles in every dimension with ragged tails, and several
vocabulary chunks in the backward pass.  The five named workloads run at
full size and are checked on every token's loss, the total loss, and dX /
dW on seeded subsets of >= 512 tokens and >= 512 vocabulary rows (the lse of
every token comes from the oracle, stored by tests/golden/make_oracle_lse.py).
"""
import math

import numpy as np
import pytest
import torch

import lm_head_cross_amd as L
import oracle
from tests.gpu_common import (TOL_GRAD_REL_L2, TOL_TOKEN_ABS, TOL_TOTAL_REL, check_full, check_rows,
                              oracle_problem, problem_of, rel_l2, run_hip, say, stored_lse)
from workloads import WORKLOADS, Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _small(key, **kw):
    base = dict(name=f"case{key}", x_std=1.0, w_std=0.05)
    base.update(kw)
    return Workload(key=key, **base)


SMALL = {
    "tiny": WORKLOADS[1],
    "ragged_softcap_mean_pad": _small(101, T=600, H=384, V=1300, Vu=1100, w_std=0.3, pad_std=30.0,
                                      softcap=7.0, reduction="mean", ignore_frac=0.1),
    "multichunk_sum_runs": _small(102, T=1000, H=512, V=3000, Vu=3000, w_std=2.0 / math.sqrt(512),
                                  ignore="runs"),
    "count_normalised": _small(103, T=777, H=256, V=2100, Vu=2049, w_std=0.1, softcap=30.0,
                               ignore_frac=0.3, normalise_by_count=True),
    "peaked": _small(104, T=300, H=256, V=4099, Vu=4099, w_std=0.4, softcap=30.0, ignore_frac=0.02,
                     labels="argmax70"),
    "fp32_head": _small(105, T=513, H=128, V=1536, Vu=1500, w_std=0.2, head_fp32=True, softcap=30.0,
                        ignore_frac=0.05),
    # H a multiple of 8 but not of 128: rows padded to 128-wide groups
    "hidden_200": _small(106, T=530, H=200, V=1800, Vu=1750, w_std=0.1, ignore_frac=0.1),
    "hidden_328_fp32_head": _small(107, T=300, H=328, V=1100, Vu=1100, w_std=0.1, head_fp32=True,
                                   softcap=30.0, ignore_frac=0.05),
    "hidden_8": _small(108, T=70, H=8, V=300, Vu=290, w_std=1.0, reduction="mean", ignore_frac=0.1),
    # the projection's 384-row head tiles: exactly one tile; two with the
    # second shifted down over all but 16 rows of the first; one row short of
    # a tile (256-row tiles)
    "vocab_384": _small(109, T=260, H=128, V=384, Vu=384, w_std=0.2, softcap=15.0, ignore_frac=0.05),
    "vocab_400": _small(110, T=300, H=256, V=420, Vu=400, w_std=0.2, ignore_frac=0.05),
    "vocab_383": _small(111, T=200, H=128, V=383, Vu=383, w_std=0.2, ignore_frac=0.05),
    # fewer than 384 usable rows with a softcap: the 256-row softcapped
    # forward and recompute tiles, a straddling tile and NaN-free padding
    "vocab_300_softcap": _small(112, T=300, H=128, V=383, Vu=300, w_std=0.5, pad_std=30.0, softcap=30.0,
                                ignore_frac=0.05),
    # hidden sizes for the 384-row dW^T tiles: one tile shifted down over all
    # but 16 rows of the first; three whole tiles and several chunks
    "hidden_400": _small(113, T=700, H=400, V=2000, Vu=1900, w_std=0.05, softcap=30.0, ignore_frac=0.1),
    "hidden_1152_chunks": _small(114, T=520, H=1152, V=5000, Vu=4800, w_std=0.03, ignore_frac=0.05),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    w = SMALL[name]
    say(f"case {name}: T={w.T} H={w.H} V={w.V} Vu={w.Vu} c={w.softcap} {w.reduction}")
    inp = make_inputs(w, argmax_device="cuda:0")
    res = run_hip(inp)
    assert res["status"] == 0
    check_full(inp, res, label=name)


DW_384 = [k for k, w in SMALL.items() if w.H >= 384]


@pytest.mark.parametrize("name", DW_384)
def test_small_full_parity_dw_tile_384(name):
    """dW on 384-row tiles of Xc^T G (stored transposed), which the library
    picks by itself only where rounds of tiles on the device favour it."""
    w = SMALL[name]
    say(f"case {name}: T={w.T} H={w.H} V={w.V} Vu={w.Vu}, dW tile 384")
    inp = make_inputs(w)
    res = run_hip(inp, dw_tile=384)
    assert res["status"] == 0
    check_full(inp, res, label=name)
    # Against 256-row dW tiles: dX takes the same kernels (bit for bit); dW
    # sums the same products over tokens in the same order.
    ref = run_hip(inp, dw_tile=256)
    for k in ("lse", "token_loss", "dX"):
        assert torch.equal(res[k], ref[k]), k
    same = torch.equal(res["dW"], ref["dW"])
    say(f"  dW bitwise equal to the 256-row tiles: {same}")
    torch.testing.assert_close(res["dW"], ref["dW"], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("dw_tile", [256, 384])
def test_all_positions_ignored_wide_hidden(dw_tile):
    """No valid token with H >= 384: dW's contraction over tokens is empty
    and every stored row must be exactly zero, on either dW tile."""
    inp = make_inputs(SMALL["hidden_400"])
    T = inp["hidden"].shape[0]
    c = dict(inp)
    c["labels"] = torch.full((T,), -100, dtype=torch.int64)
    res = run_hip(c, dw_tile=dw_tile)
    assert res["status"] == 0 and res["loss"] == 0.0
    assert torch.all(res["dX"] == 0) and torch.all(res["dW"] == 0)


def test_fp32_head_handed_over_directly():
    """An fp32 head passed to the calls as fp32.  Staged (the default: each
    call rounds the usable rows into the workspace): bit for bit the
    pre-rounded bf16 head's results.  Rounded on load (inside the GEMMs'
    tile loads): the oracle's result, and the pre-rounded head's within the
    tolerances (it takes 256-row tiles where the bf16 head takes 384-row
    ones, so the per-tile lse partials round differently).  Padding rows are
    never read in either mode (NaN there changes nothing, bit for bit)."""
    w = SMALL["fp32_head"]
    inp = make_inputs(w, argmax_device="cuda:0")
    b = run_hip(inp)
    a = run_hip(inp, fp32_head_direct=True)
    check_full(inp, a, label="fp32 head staged")
    assert a["loss"] == b["loss"]
    for k in ("lse", "token_loss", "dX", "dW"):
        assert torch.equal(a[k], b[k]), k
    r = run_hip(inp, fp32_head_direct=True, round_on_load=True)
    check_full(inp, r, label="fp32 head rounded on load")
    assert abs(r["loss"] - b["loss"]) <= TOL_TOTAL_REL * abs(b["loss"])
    assert (r["token_loss"] - b["token_loss"]).abs().max().item() <= TOL_TOKEN_ABS
    for k in ("dX", "dW"):
        assert rel_l2(r[k].double().numpy(), b[k].double().numpy()) <= TOL_GRAD_REL_L2, k
    poisoned = dict(inp)
    W = inp["weight"].clone()
    W[w.Vu:] = float("nan")
    poisoned["weight"] = W
    for ref, rol in ((a, False), (r, True)):
        c = run_hip(poisoned, fp32_head_direct=True, round_on_load=rol)
        for k in ("lse", "token_loss", "dX", "dW"):
            assert torch.equal(ref[k], c[k]), (k, rol)


def _tie_head(w, seed):
    """An fp32 head whose every element is an exact tie between two bf16
    values (low 16 bits 0x8000), half with an even and half with an odd kept
    bit, plus some values that round up or down: round to nearest even is
    the only rounding that gives the pre-rounded head's values."""
    g = torch.Generator().manual_seed(seed)
    base = (torch.randn(w.V, w.H, generator=g) * w.w_std).to(torch.bfloat16).to(torch.float32)
    bits = base.view(torch.int32)
    tie = bits | 0x8000
    low = torch.randint(1, 0x10000, (w.V, w.H), generator=g, dtype=torch.int32)
    pick = torch.rand(w.V, w.H, generator=g) < 0.8
    return torch.where(pick, tie, bits | low).view(torch.float32)


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_fp32_head_rounding_on_load_is_the_bf16_cast(softcap):
    """With fewer than 384 usable rows and at most 256 tokens both paths run
    the same 256-row tiles, so the fp32 head rounded on its way into LDS
    (FLCE_FLAG_ROUND_HEAD_ON_LOAD) must
    give, bit for bit, the results of the head rounded beforehand by
    flce_round_to_bf16 (torch's cast, checked against the oracle's rounding
    below): every head element is a rounding tie or near one."""
    w = _small(120, T=250, H=256, V=383, Vu=350, w_std=0.3, ignore_frac=0.05, softcap=softcap)
    inp = dict(make_inputs(w))
    inp["weight"] = _tie_head(w, 5)
    a = run_hip(inp, fp32_head_direct=True, round_on_load=True)
    b = run_hip(inp)
    assert a["status"] == b["status"] == 0
    assert a["loss"] == b["loss"]
    for k in ("lse", "token_loss", "dX", "dW"):
        assert torch.equal(a[k], b[k]), k
    check_full(inp, a, label=f"fp32 tie head, c={softcap}")


def test_grad_out_scaling():
    w = SMALL["ragged_softcap_mean_pad"]
    inp = make_inputs(w)
    res = run_hip(inp, grad_out=-2.5)
    check_full(inp, res, grad_out=-2.5, label="grad_out=-2.5")


def test_dweight_columns_sum_to_zero():
    """Without a softcap, sum_v G[t, v] = (g/D) (sum_v p - 1) = 0 for every
    token, so every column of dW = G^T X sums to zero over the head rows.  G
    is stored in bf16 (relative rounding <= 2^-9), and sum_v |G[t, v]| =
    2 (1 - p_y) g/D <= 2 g/D, so |sum_v dW[v, h]| <= 2^-8 (g/D) sum_t |X[t, h]|
    over valid tokens, plus fp32 accumulation slack."""
    w = SMALL["multichunk_sum_runs"]
    inp = make_inputs(w)
    assert w.softcap == 0.0 and w.reduction == "sum"
    g = 1.75
    res = run_hip(inp, grad_out=g)
    colsum = res["dW"].double().sum(0).numpy()
    valid = (inp["labels"] != inp["ignore_index"]).numpy()
    X = inp["hidden"].double().numpy()[valid]
    bound = 2.0 ** -8 * g * np.abs(X).sum(0)
    scale = np.abs(res["dW"].double().numpy()).sum(0)
    say(f"max |colsum| / bound = {np.max(np.abs(colsum) / bound):.3g}")
    assert np.all(np.abs(colsum) <= bound + 1e-5 * scale + 1e-6)


def test_deterministic_repeat():
    inp = make_inputs(SMALL["multichunk_sum_runs"])
    a = run_hip(inp)
    b = run_hip(inp)
    assert a["loss"] == b["loss"]
    for k in ("lse", "token_loss", "dX", "dW"):
        assert torch.equal(a[k], b[k]), k


def test_padding_rows_never_read():
    """NaN in the head rows past unpadded_vocab changes nothing, bit for bit."""
    inp = make_inputs(SMALL["ragged_softcap_mean_pad"])
    a = run_hip(inp)
    poisoned = dict(inp)
    W = inp["weight"].clone()
    W[inp["unpadded_vocab"]:] = float("nan")
    poisoned["weight"] = W
    b = run_hip(poisoned)
    assert a["loss"] == b["loss"]
    for k in ("lse", "token_loss", "dX", "dW"):
        assert torch.equal(a[k], b[k]), k
    assert torch.all(b["dW"][inp["unpadded_vocab"]:] == 0)


@pytest.mark.parametrize("name", ["hidden_200", "hidden_328_fp32_head"])
def test_unaligned_hidden_equals_zero_padded_problem(name):
    """H not a multiple of 128 gives, bit for bit, the results of the same
    problem with X and W extended by zero columns to the next multiple of 128
    (the padded problem's extra dX and dW columns are exactly 0); with the
    fp32 head handed over directly, the staging kernel's rounding is the
    rounding kernel's."""
    w = SMALL[name]
    inp = make_inputs(w)
    H = w.H
    Hp = (H + 127) // 128 * 128
    direct = inp["weight"].dtype == torch.float32
    a = run_hip(inp, fp32_head_direct=direct)
    padded = dict(inp)
    padded["hidden"] = torch.nn.functional.pad(inp["hidden"], (0, Hp - H))
    padded["weight"] = torch.nn.functional.pad(inp["weight"], (0, Hp - H))
    b = run_hip(padded)
    assert a["status"] == b["status"] == 0
    assert a["loss"] == b["loss"]
    for k in ("lse", "token_loss"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["dX"], b["dX"][:, :H])
    assert torch.equal(a["dW"], b["dW"][:, :H])
    assert torch.all(b["dX"][:, H:] == 0) and torch.all(b["dW"][:, H:] == 0)


def _custom(inp, labels, **kw):
    out = dict(inp)
    out["labels"] = torch.as_tensor(labels, dtype=torch.int64)
    out.update(kw)
    return out


@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_all_positions_ignored(reduction):
    inp = make_inputs(WORKLOADS[1])
    T = inp["hidden"].shape[0]
    c = _custom(inp, np.full(T, -100), reduction=reduction)
    res = run_hip(c)
    if reduction == "sum":
        assert res["loss"] == 0.0
    else:
        assert math.isnan(res["loss"])
    assert torch.all(res["dX"] == 0) and torch.all(res["dW"] == 0)
    assert torch.all(res["lse"] == 0) and torch.all(res["token_loss"] == 0)


def test_single_token_and_vocab_edges():
    inp = make_inputs(SMALL["ragged_softcap_mean_pad"])
    T = inp["hidden"].shape[0]
    Vu = inp["unpadded_vocab"]
    lab = np.full(T, -100)
    lab[T - 1] = Vu - 1
    res = run_hip(_custom(inp, lab))
    check_full(_custom(inp, lab), res, label="single token, last usable row")
    lab = np.full(T, -100)
    lab[0] = 0
    lab[255] = 255
    lab[256] = 256
    lab[T - 1] = Vu - 1
    check_full(_custom(inp, lab), run_hip(_custom(inp, lab)), label="tile edges")


def test_one_token_problem():
    inp = make_inputs(WORKLOADS[1])
    one = dict(inp)
    one["hidden"] = inp["hidden"][5:6].contiguous()
    one["labels"] = torch.tensor([17])
    check_full(one, run_hip(one), label="T=1")


def test_ignore_index_inside_vocabulary():
    inp = make_inputs(WORKLOADS[1])
    lab = inp["labels"].numpy().copy()
    lab[lab == -100] = 3
    lab[:5] = 3
    c = _custom(inp, lab, ignore_index=3)
    check_full(c, run_hip(c), label="ignore_index=3")


def test_out_of_range_labels_flagged_and_skipped():
    inp = make_inputs(WORKLOADS[1])
    lab = inp["labels"].numpy().copy()
    bad = lab.copy()
    bad[[1, 7]] = [1000, -5]
    res = run_hip(_custom(inp, bad))
    assert res["status"] == 1
    ref = lab.copy()
    ref[[1, 7]] = -100
    check_full(_custom(inp, ref), res, label="bad labels as ignored")


def test_empty_batch():
    d = torch.device("cuda:0")
    p = L.make_problem(0, 128, 1000, reduction="mean")
    X = torch.empty((0, 128), dtype=torch.bfloat16, device=d)
    W = torch.randn(1000, 128, device=d).to(torch.bfloat16)
    y = torch.empty(0, dtype=torch.int64, device=d)
    loss = torch.zeros((), device=d)
    lse = torch.empty(0, device=d)
    L.flce_forward(p, X, W, y, loss, lse)
    dW = torch.full((1000, 128), 7.0, device=d)
    L.flce_backward(p, X, W, y, lse, torch.ones((), device=d), torch.empty_like(X), dW)
    torch.cuda.synchronize()
    assert math.isnan(loss.item())
    assert torch.all(dW == 0)


def test_round_to_bf16_matches_oracle_rounding():
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.standard_normal(100003).astype(np.float32),
                        ((rng.integers(0, 0x7F7F, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40], dtype=np.float32)])
    for arr in (a, a[:100001]):  # vector and scalar kernel paths
        src = torch.from_numpy(arr.copy()).to("cuda:0")
        got = L.flce_round_to_bf16(src).cpu().double().numpy()
        assert np.array_equal(got, oracle.round_fp32_to_bf16(arr))


# ---------------------------------------------------------------------------
# Full-size workloads, sampled checks
# ---------------------------------------------------------------------------


def test_workload3_fp32_head_direct_staged_matches_pre_rounded():
    """Softcapped padded head (fp32 head, V=262144, Vu=256000) at full size:
    handing the fp32 head over directly (staged by each call) is
    bit-identical to rounding it first (the rounded path, and the head
    rounded on load, are checked against the oracle below)."""
    w = WORKLOADS[3]
    inp = make_inputs(w)
    rows = np.arange(0, w.T, 97)
    vrows = np.arange(0, w.V, 1021)
    a = run_hip(inp, dx_rows=rows, dw_rows=vrows, fp32_head_direct=True)
    b = run_hip(inp, dx_rows=rows, dw_rows=vrows)
    assert a["status"] == 0 and a["loss"] == b["loss"]
    for k in ("lse", "token_loss", "dX", "dW"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("key,on_load", [(2, False), (3, False), (3, True), (4, False), (5, False)])
def test_workload_full_size(key, on_load):
    """Full-size workloads; workload 3's fp32 head also handed over directly
    and rounded to bf16 inside the GEMMs' tile loads."""
    w = WORKLOADS[key]
    say(f"workload {key}: {w.name}" + (" (fp32 head rounded on load)" if on_load else ""))
    inp = make_inputs(w, argmax_device="cuda:0")
    y = inp["labels"].numpy()
    tok, voc = sample_rows(w, y)
    res = run_hip(inp, dx_rows=tok, dw_rows=voc, keep_device=True, fp32_head_direct=on_load,
                  round_on_load=on_load)
    assert res["status"] == 0
    if w.V > w.Vu:
        assert res["dW_dev"][w.Vu:].abs().max().item() == 0.0
    valid = y != -100
    assert torch.all(res["dX_dev"][torch.from_numpy(~valid).to("cuda:0")] == 0)
    del res["dW_dev"], res["dX_dev"]
    torch.cuda.empty_cache()

    X = oracle.to_f64(inp["hidden"])
    W = oracle.head_values(inp["weight"])[: w.Vu]
    p = oracle_problem(inp)
    D = oracle.divisor(p, int(valid.sum()))
    lse_all = stored_lse(key)
    ref = oracle.loss_from_lse(lse_all, oracle.label_logits(X, W, y, p), y, p)
    ref_tl, ref_loss = ref.token_loss, ref.loss
    assert ref.D == D
    tl_err = np.abs(res["token_loss"].double().numpy() - ref_tl).max()
    say(f"  loss gpu={res['loss']:.9g} ref={ref_loss:.9g} rel={abs(res['loss'] - ref_loss) / abs(ref_loss):.3g}"
        f" max|dl|={tl_err:.3g}")
    assert tl_err <= TOL_TOKEN_ABS
    assert abs(res["loss"] - ref_loss) <= TOL_TOTAL_REL * abs(ref_loss)
    lse_gpu = res["lse"].double().numpy()
    assert np.abs(lse_gpu[valid] - lse_all[valid]).max() <= TOL_TOKEN_ABS

    tl_s, lse_s, dX_s = oracle.token_rows(X, W, y, tok, p, D)
    # The stored lse must be the live oracle's (same inputs on this machine).
    vs = valid[tok]
    np.testing.assert_allclose(lse_s[vs], lse_all[tok][vs], rtol=1e-12)
    e_dx = rel_l2(res["dX"].double().numpy(), dX_s)
    dW_r = oracle.weight_rows(X, W, y, voc, lse_all, p, D)
    e_dw = rel_l2(res["dW"].double().numpy(), dW_r)
    say(f"  dX relL2 over {len(tok)} rows = {e_dx:.3g}; dW relL2 over {len(voc)} rows = {e_dw:.3g}")
    assert e_dx <= TOL_GRAD_REL_L2
    assert e_dw <= TOL_GRAD_REL_L2
    wx = check_rows(res["dX"].double().numpy(), dX_s, "dX")
    ww = check_rows(res["dW"].double().numpy(), dW_r, "dW")
    say(f"  worst row error / row scale: dX {wx:.3g}, dW {ww:.3g}")


def test_no_logits_sized_allocation():
    """Forward + backward at the llama3-8b head shape with the outputs already
    allocated: the call's extra device memory (the workspace the binding
    allocates) stays below one bf16 [T, Vu] logits buffer."""
    w = WORKLOADS[2]
    d = torch.device("cuda:0")
    inp = make_inputs(w, device="cuda:0")
    p = L.make_problem(w.T, w.H, w.V, w.Vu, w.softcap, inp["ignore_index"], w.reduction, inp["num_label_tokens"])
    loss = torch.empty((), device=d)
    lse = torch.empty(w.T, device=d)
    dX = torch.empty_like(inp["hidden"])
    dW = torch.empty((w.V, w.H), device=d)
    g = torch.ones((), device=d)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(d)
    base = torch.cuda.memory_allocated(d)
    L.flce_forward(p, inp["hidden"], inp["weight"], inp["labels"], loss, lse)
    L.flce_backward(p, inp["hidden"], inp["weight"], inp["labels"], lse, g, dX, dW)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated(d) - base
    say(f"  extra device memory {extra / 2**20:.1f} MiB, workspace {L.flce_workspace_size(p) / 2**20:.1f} MiB, "
        f"bf16 [T, Vu] {w.T * w.Vu * 2 / 2**20:.1f} MiB")
    assert extra < w.T * w.Vu * 2
    assert math.isfinite(loss.item())


@pytest.mark.parametrize("softcap", [0.0, 30.0])
def test_single_usable_row(softcap):
    """Vu = 1 (the degenerate softmax over one row): every valid token's loss,
    and both gradients, are exactly 0 mathematically (softmax = one-hot).  In
    fp32 the kernels reach them up to rounding: |loss_t| and every gradient
    element stay below 1e-5 of their natural scales, padding rows of dW are
    exactly 0 and the oracle gives exact zeros."""
    w = _small(121, T=300, H=128, V=8, Vu=1, w_std=0.5, pad_std=10.0, softcap=softcap, ignore_frac=0.1)
    inp = dict(make_inputs(w))
    y = inp["labels"].clone()
    y[y != -100] = 0
    inp["labels"] = y
    X, W = oracle.to_f64(inp["hidden"]), oracle.head_values(inp["weight"])
    ref = oracle.forward(X, W, y.numpy(), oracle_problem(inp))
    rdX, rdW = oracle.backward(X, W, y.numpy(), oracle_problem(inp))
    assert ref.loss == 0.0 and not rdX.any() and not rdW.any()
    res = run_hip(inp)
    assert res["status"] == 0
    assert res["token_loss"].abs().max().item() <= 1e-5
    assert abs(res["loss"]) <= 1e-5 * ref.n_valid
    wmax = inp["weight"][:1].float().abs().max().item()
    xmax = inp["hidden"].float().abs().max().item()
    assert res["dX"].float().abs().max().item() <= 1e-5 * wmax
    assert res["dW"][:1].abs().max().item() <= 1e-5 * xmax * ref.n_valid
    assert torch.all(res["dW"][1:] == 0)


@pytest.mark.parametrize("name,direct", [("fp32_head", True), ("hidden_328_fp32_head", True),
                                         ("hidden_200", False), ("multichunk_sum_runs", False)])
def test_backward_reuses_the_forward_staged_head(name, direct):
    """FLCE_FLAG_HEAD_STAGED: the backward reads the head copy that the
    forward staged in the same workspace.  With a staged copy (an fp32 head
    handed over directly, or H not a multiple of 128) the backward is handed
    a NaN head and must not read it; without one the bit changes nothing.
    Either way the results equal the unflagged run bit for bit."""
    d = torch.device("cuda:0")
    inp = make_inputs(SMALL[name])
    ref = run_hip(inp, fp32_head_direct=direct)
    X, W, y = inp["hidden"].to(d), inp["weight"].to(d), inp["labels"].to(d)
    if W.dtype == torch.float32 and not direct:
        W = L.flce_round_to_bf16(W)
    p = problem_of(inp, W.dtype, head_staged=True)
    T, H, V = p.num_tokens, p.hidden, p.vocab
    staged = W.dtype == torch.float32 or H % 128 != 0
    ws = L.alloc_workspace(p, d)
    loss = torch.empty((), dtype=torch.float32, device=d)
    lse = torch.empty(T, dtype=torch.float32, device=d)
    tl = torch.empty(T, dtype=torch.float32, device=d)
    L.flce_forward(p, X, W, y, loss, lse, tl, None, ws)
    Wb = torch.full_like(W, float("nan")) if staged else W
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=d)
    L.flce_backward(p, X, Wb, y, lse, torch.tensor(1.0, device=d), dX, dW, None, ws)
    torch.cuda.synchronize()
    assert loss.item() == ref["loss"]
    assert torch.equal(lse.cpu(), ref["lse"]) and torch.equal(tl.cpu(), ref["token_loss"])
    assert torch.equal(dX.cpu(), ref["dX"]) and torch.equal(dW.cpu(), ref["dW"])


def test_two_streams_at_once_equal_one_after_the_other():
    """The library keeps no state between calls: two problems enqueued
    interleaved on two streams (each with its own workspace), with no
    synchronisation between them, give bit for bit the results of running
    them one after the other on the default stream."""
    d = torch.device("cuda:0")
    cases = [make_inputs(SMALL["multichunk_sum_runs"]), make_inputs(SMALL["hidden_400"])]
    refs = [run_hip(inp) for inp in cases]
    runs = []
    for inp in cases:
        X, W, y = inp["hidden"].to(d), inp["weight"].to(d), inp["labels"].to(d)
        p = problem_of(inp)
        T, H, V = p.num_tokens, p.hidden, p.vocab
        runs.append(dict(p=p, X=X, W=W, y=y, ws=L.alloc_workspace(p, d),
                         loss=torch.empty((), device=d), lse=torch.empty(T, device=d),
                         tl=torch.empty(T, device=d), g=torch.tensor(1.0, device=d),
                         dX=torch.empty_like(X), dW=torch.empty((V, H), device=d)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for r, s in zip(runs, streams):
        L.flce_forward(r["p"], r["X"], r["W"], r["y"], r["loss"], r["lse"], r["tl"], None, r["ws"], stream=s)
    for r, s in zip(runs, streams):
        L.flce_backward(r["p"], r["X"], r["W"], r["y"], r["lse"], r["g"], r["dX"], r["dW"], None, r["ws"],
                        stream=s)
    torch.cuda.synchronize()
    for r, ref in zip(runs, refs):
        assert r["loss"].item() == ref["loss"]
        assert torch.equal(r["lse"].cpu(), ref["lse"]) and torch.equal(r["tl"].cpu(), ref["token_loss"])
        assert torch.equal(r["dX"].cpu(), ref["dX"]) and torch.equal(r["dW"].cpu(), ref["dW"])
