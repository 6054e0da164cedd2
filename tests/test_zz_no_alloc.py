"""flce_forward_noalloc: the forward pass on the library's own fixed scratch
(no workspace argument, no allocation), for callers that cannot allocate.

Checked through the C ABI against flce_forward on a caller workspace: two
calls in a row, the second on a smaller problem (the scratch keeps the first
call's contents), each bit-identical in loss, lse and per-token loss; the
first is the llama3-8b head's forward (T=4096, H=4096, V=128256), near the
scratch's 64 MiB limit.  A problem whose forward needs more than the limit is
refused before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import lm_head_cross_amd as L
from lm_head_cross_amd import _lib
from tests.gpu_common import say
from workloads import WORKLOADS, Workload, make_inputs


SCRATCH_LIMIT = 64 << 20


def _noalloc(problem, X, W, y, loss, lse, tl, st):
    fn = _lib.load().flce_forward_noalloc
    return fn(ctypes.byref(problem), ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(W.data_ptr()),
              ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(loss.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
              ctypes.c_void_p(tl.data_ptr()), ctypes.c_void_p(st.data_ptr()),
              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _both(inp):
    d = torch.device("cuda:0")
    X, W, y = inp["hidden"].to(d), inp["weight"].to(d), inp["labels"].to(d)
    if W.dtype == torch.float32:
        W = L.flce_round_to_bf16(W)
    T, H = X.shape
    p = L.make_problem(T, H, W.shape[0], inp["unpadded_vocab"], inp["softcap"], inp["ignore_index"],
                       inp["reduction"], inp["num_label_tokens"])
    out = []
    for which in ("workspace", "noalloc"):
        loss = torch.full((), float("nan"), device=d)
        lse = torch.full((T,), float("nan"), device=d)
        tl = torch.full((T,), float("nan"), device=d)
        st = torch.zeros((), dtype=torch.int32, device=d)
        if which == "workspace":
            L.flce_forward(p, X, W, y, loss, lse, tl, st)
        else:
            code = _noalloc(p, X, W, y, loss, lse, tl, st)
            assert code == 0, _lib.status_string(code)
        torch.cuda.synchronize()
        out.append((loss.cpu(), lse.cpu(), tl.cpu(), int(st.item())))
    return out


@pytest.mark.gpu
def test_noalloc_forward_equals_workspace_forward_twice():
    big = WORKLOADS[2]
    small = Workload(key=113, name="small", T=300, H=256, V=1300, Vu=1100, x_std=1.0, w_std=0.3, pad_std=30.0,
                     softcap=30.0, reduction="mean", ignore_frac=0.1)
    for w in (big, small):
        say(f"noalloc case: T={w.T} H={w.H} V={w.V} Vu={w.Vu} c={w.softcap}")
        (la, sa, ta, qa), (lb, sb, tb, qb) = _both(make_inputs(w))
        assert qa == qb == 0
        assert torch.isfinite(la) and torch.equal(la, lb)
        assert torch.equal(sa, sb) and torch.equal(ta, tb)
        say(f"  loss {la.item():.9g} identical on both entry points")


@pytest.mark.skipif(torch.cuda.is_available(), reason="host-side check with fake device addresses: it runs "
                                                      "only where no GPU is present")
@pytest.mark.parametrize("T,H,V,fp32_head", [(16384, 4096, 32000, False), (4096, 4000, 128256, True)])
def test_noalloc_refuses_problems_beyond_the_scratch(T, H, V, fp32_head):
    """Host-side refusal, no GPU needed: the gathered hidden rows alone are
    128 MiB in the first problem; the second (H not a multiple of 128)
    stages a zero-padded bf16 copy of the head (1 GiB).  Fake device
    addresses: nothing is launched or read."""
    p = L.make_problem(T, H, V, weight_dtype=torch.float32 if fp32_head else torch.bfloat16)
    fake = ctypes.c_void_p(1 << 20)
    fn = _lib.load().flce_forward_noalloc
    code = fn(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, ctypes.c_void_p(0))
    assert code == _lib.FLCE_ERR_WORKSPACE

