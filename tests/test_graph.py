"""The fused path under HIP graph capture (torch.cuda.CUDAGraph), and the
launch trace's kind filter.

The library allocates nothing, sets no memory with memset nodes and never
synchronises the host, so a forward + backward pass can be captured once and
replayed.  Every replay must equal the eager result bit for bit, also after
the inputs are overwritten in place between replays (the graph recomputes).
"""
import pytest
import torch

import lm_head_cross_amd as L
from tests.gpu_common import problem_of, say
from tests.test_parity import SMALL
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _buffers(inp, d, direct=False, **opts):
    """Device buffers of one problem; ``direct`` hands an fp32 head to the
    calls as fp32 (else it is rounded first); ``opts`` go to the problem."""
    X = inp["hidden"].to(d)
    W = inp["weight"].to(d)
    y = inp["labels"].to(d)
    if W.dtype == torch.float32 and not direct:
        W = L.flce_round_to_bf16(W)
    p = problem_of(inp, W.dtype, **opts)
    T, H, V = p.num_tokens, p.hidden, p.vocab
    out = {
        "loss": torch.empty((), dtype=torch.float32, device=d),
        "lse": torch.empty(T, dtype=torch.float32, device=d),
        "tl": torch.empty(T, dtype=torch.float32, device=d),
        "st": torch.zeros((), dtype=torch.int32, device=d),
        "g": torch.tensor(1.25, dtype=torch.float32, device=d),
        "dX": torch.empty_like(X),
        "dW": torch.empty((V, H), dtype=torch.float32, device=d),
        "ws": L.alloc_workspace(p, d),
    }
    return p, X, W, y, out


def _step(p, X, W, y, o):
    L.flce_forward(p, X, W, y, o["loss"], o["lse"], o["tl"], o["st"], o["ws"])
    L.flce_backward(p, X, W, y, o["lse"], o["g"], o["dX"], o["dW"], o["st"], o["ws"])


def _snapshot(o):
    return {k: o[k].clone() for k in ("loss", "lse", "tl", "dX", "dW", "st")}


GRAPH_CASES = {
    "multichunk_sum_runs": {},
    "ragged_softcap_mean_pad": {},
    # the staging pass inside the graph, its copy reused by the backward
    "fp32_head": dict(direct=True, head_staged=True),
    # dW on 384-row tiles of Xc^T G
    "hidden_1152_chunks": dict(dw_tile=384),
}


@pytest.mark.parametrize("name", list(GRAPH_CASES))
def test_captured_step_replays_match_eager(name):
    d = torch.device("cuda:0")
    inp = make_inputs(SMALL[name])
    opts = GRAPH_CASES[name]
    say(f"graph case {name} {opts}")
    p, X, W, y, o = _buffers(inp, d, **opts)
    _step(p, X, W, y, o)  # eager (also warms up lazily initialised state)
    torch.cuda.synchronize()
    eager = _snapshot(o)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(p, X, W, y, o)
    torch.cuda.synchronize()

    # a second input set, eager, in buffers of its own
    inp2 = make_inputs(SMALL[name])
    X2 = (inp2["hidden"].float() * 0.5).to(torch.bfloat16).to(d)
    p2, _, _, _, o2 = _buffers(inp, d, **opts)
    _step(p2, X2, W, y, o2)
    torch.cuda.synchronize()
    eager2 = _snapshot(o2)

    for rep in range(3):
        for k in ("loss", "lse", "tl", "dX", "dW"):
            o[k].fill_(float("nan")) if o[k].is_floating_point() else o[k].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(o)
        for k in ("loss", "lse", "tl", "dX", "dW"):
            assert torch.equal(got[k], eager[k]), (rep, k)
        assert int(got["st"].item()) == 0
        # eager work between replays
        _step(p2, X2, W, y, o2)
        torch.cuda.synchronize()

    # overwrite the captured input in place: the replay recomputes
    X.copy_(X2)
    g.replay()
    torch.cuda.synchronize()
    got = _snapshot(o)
    for k in ("loss", "lse", "tl", "dX", "dW"):
        assert torch.equal(got[k], eager2[k]), ("new input", k)


def test_launch_trace_kind_filter():
    """The launch trace records only the selected kinds, and after stop()
    every kind again (the bench times its dominant kernel this way)."""
    d = torch.device("cuda:0")
    inp = make_inputs(SMALL["multichunk_sum_runs"])
    p, X, W, y, o = _buffers(inp, d)
    _step(p, X, W, y, o)
    torch.cuda.synchronize()
    tr = L.LaunchTrace(capacity=256, kinds=["dgrad"]).start()
    _step(p, X, W, y, o)
    torch.cuda.synchronize()
    tr.stop()
    rec = tr.records()
    assert rec and all(k == "dgrad" for k, _, _ in rec)
    assert all(ms > 0 and fl > 0 for _, ms, fl in rec)
    full = L.LaunchTrace(capacity=256).start()
    _step(p, X, W, y, o)
    torch.cuda.synchronize()
    full.stop()
    kinds = {k for k, _, _ in full.records()}
    assert {"proj_lse", "recompute_g", "dgrad", "compact", "gather"} <= kinds
    assert sum(k == "dgrad" for k, _, _ in full.records()) == len(rec)
