"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the CPU oracle to the stated tolerances.

Tolerances (fp32 logits / CE on bf16 inputs, bf16 gradient staging):
  per-token loss  |gpu - ref| <= 2e-3
  total loss      |gpu - ref| <= 1e-4 |ref|
  dHidden, dWeight  ||gpu - ref||_2 <= 1e-2 ||ref||_2 over the checked rows
and, beside that aggregate, every checked row on its own:
  ||gpu_r - ref_r||_2 <= 5e-2 max(||ref_r||_2, 5e-2 rms_r ||ref_r||_2)
i.e. five times the aggregate bound per row, with rows whose norm is under
5% of the rows' rms held to that floor (rows of near-total cancellation,
whose relative error the bf16 rounding of G can inflate).  A few rows wrong
by 10% or more fail it even where the aggregate over hundreds of rows would
not; rows whose reference is exactly zero must be exactly zero.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

import lm_head_cross_amd as L
import oracle

TOL_TOKEN_ABS = 2e-3
TOL_TOTAL_REL = 1e-4
TOL_GRAD_REL_L2 = 1e-2
TOL_GRAD_ROW = 5e-2
ROW_FLOOR = 5e-2
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def problem_of(inp, weight_dtype=torch.bfloat16, round_on_load=False, dw_tile=None, head_staged=False):
    X, W = inp["hidden"], inp["weight"]
    return L.make_problem(X.shape[0], X.shape[1], W.shape[0], inp["unpadded_vocab"], inp["softcap"],
                          inp["ignore_index"], inp["reduction"], inp["num_label_tokens"], weight_dtype,
                          round_head_on_load=round_on_load, dw_tile=dw_tile, head_staged=head_staged)


def run_hip(inp, grad_out=1.0, dx_rows=None, dw_rows=None, keep_device=False, fp32_head_direct=False,
            round_on_load=False, dw_tile=None, head_staged=False):
    """Forward + backward through the C ABI.  Returns CPU results; dX / dW
    are restricted to the given rows (all when None).  An fp32 head is rounded
    by flce_round_to_bf16 first, or with ``fp32_head_direct`` handed to the
    calls as fp32 (the library stages the rounded rows itself, or with
    ``round_on_load`` rounds them inside the GEMMs' tile loads).  ``dw_tile``
    fixes the dW contraction's tile (256 or 384 rows); ``head_staged`` lets
    the backward reuse the forward's staged head (same workspace)."""
    d = dev()
    X = inp["hidden"].to(d)
    W = inp["weight"].to(d)
    y = inp["labels"].to(d)
    direct = fp32_head_direct and W.dtype == torch.float32
    if W.dtype == torch.float32 and not direct:
        W = L.flce_round_to_bf16(W)
    p = problem_of(inp, torch.float32 if direct else torch.bfloat16, round_on_load=direct and round_on_load,
                   dw_tile=dw_tile, head_staged=head_staged)
    T, H, V = p.num_tokens, p.hidden, p.vocab
    ws = L.alloc_workspace(p, d)
    loss = torch.empty((), dtype=torch.float32, device=d)
    lse = torch.empty(T, dtype=torch.float32, device=d)
    tl = torch.empty(T, dtype=torch.float32, device=d)
    st = torch.zeros((), dtype=torch.int32, device=d)
    L.flce_forward(p, X, W, y, loss, lse, tl, st, ws)
    g = torch.tensor(grad_out, dtype=torch.float32, device=d)
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=d)
    L.flce_backward(p, X, W, y, lse, g, dX, dW, st, ws)
    torch.cuda.synchronize()
    out = {
        "loss": loss.item(),
        "lse": lse.cpu(),
        "token_loss": tl.cpu(),
        "status": int(st.item()),
        "dX": (dX if dx_rows is None else dX[torch.as_tensor(dx_rows, device=d)]).cpu(),
        "dW": (dW if dw_rows is None else dW[torch.as_tensor(dw_rows, device=d)]).cpu(),
    }
    if keep_device:
        out["dW_dev"] = dW
        out["dX_dev"] = dX
    return out


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    diff = np.linalg.norm(a - b)
    return diff / nb if nb > 0 else diff


def check_rows(got, ref, label=""):
    """Per-row bound beside the aggregate rel-L2 (see the module docstring).
    Returns the largest row error relative to its bound's scale."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.linalg.norm(got - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    rms = math.sqrt(float(np.mean(nrm ** 2))) if len(nrm) else 0.0
    scale = np.maximum(nrm, ROW_FLOOR * rms)
    worst = float(np.max(np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), 0.0), initial=0.0))
    bad = np.nonzero(err > TOL_GRAD_ROW * scale)[0]
    assert len(bad) == 0, (label, "rows over the per-row bound", bad[:10].tolist(), worst)
    return worst


def oracle_problem(inp):
    return oracle.Problem(inp["unpadded_vocab"], inp["softcap"], inp["ignore_index"], inp["reduction"],
                          inp["num_label_tokens"])


def check_full(inp, res, grad_out=1.0, label=""):
    """Whole-problem comparison for shapes the oracle evaluates densely."""
    X = oracle.to_f64(inp["hidden"])
    W = oracle.head_values(inp["weight"])
    y = inp["labels"].numpy()
    p = oracle_problem(inp)
    fw = oracle.forward(X, W, y, p)
    dX, dW = oracle.backward(X, W, y, p, grad_out=grad_out)
    tl_err = np.abs(res["token_loss"].double().numpy() - fw.token_loss).max(initial=0.0)
    say(f"[{label}] loss gpu={res['loss']:.8g} ref={fw.loss:.8g} max|dl|={tl_err:.3g} "
        f"dX relL2={rel_l2(res['dX'].double().numpy(), dX):.3g} dW relL2={rel_l2(res['dW'].double().numpy(), dW):.3g}")
    assert tl_err <= TOL_TOKEN_ABS, (label, tl_err)
    if np.isnan(fw.loss):
        assert np.isnan(res["loss"]), label
    else:
        assert abs(res["loss"] - fw.loss) <= TOL_TOTAL_REL * abs(fw.loss) + 1e-6, (label, res["loss"], fw.loss)
    assert rel_l2(res["dX"].double().numpy(), dX) <= TOL_GRAD_REL_L2, label
    assert rel_l2(res["dW"].double().numpy(), dW) <= TOL_GRAD_REL_L2, label
    wx = check_rows(res["dX"].double().numpy(), dX, label + " dX")
    ww = check_rows(res["dW"].double().numpy(), dW, label + " dW")
    say(f"[{label}] worst row error / row scale: dX {wx:.3g}, dW {ww:.3g} (bound {TOL_GRAD_ROW})")
    valid = y != inp["ignore_index"]
    # Exact structure: ignored rows of dX and padding rows of dW are zero;
    # lse / token loss are zero at ignored positions.
    assert torch.all(res["dX"][torch.from_numpy(~valid)] == 0), label
    assert torch.all(res["dW"][p.unpadded_vocab:] == 0), label
    assert torch.all(res["token_loss"][torch.from_numpy(~valid)] == 0), label
    np.testing.assert_allclose(res["lse"].double().numpy()[valid], fw.lse[valid], rtol=0, atol=TOL_TOKEN_ABS)
    return fw


def stored_lse(key):
    path = os.path.join(GOLDEN, f"oracle_lse_w{key}.npy")
    return np.load(path, allow_pickle=False)
