"""A seeded sweep of random small problems against the oracle, element by
element (GPU).  Each case draws its shape (any T up to 1200, H a multiple of 8
up to 1200, 2 <= Vu <= 5000 with up to 63 padding rows), softcap, reduction,
ignore pattern and head dtype, and the call's options (dW tile, an fp32 head
handed over directly, reuse of the forward's staged head), so that tile
edges, ragged tails and option combinations that the named cases do not
spell out are met too.  Same tolerances as tests/test_parity.py."""
import math

import numpy as np
import pytest

from tests.gpu_common import check_full, run_hip, say
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw_case(i):
    rng = np.random.default_rng(7000 + i)
    T = int(rng.choice([1, 63, 255, 256, 257, 383, 385, 640] + [int(x) for x in rng.integers(1, 1201, 4)]))
    H = int(rng.integers(1, 151)) * 8
    Vu = int(rng.integers(2, 5001))
    V = Vu + int(rng.integers(0, 64))
    ignore_frac = float(rng.choice([0.0, 0.05, 0.3, 0.9])) if T >= 50 else 0.0
    w = Workload(
        key=500 + i, name=f"sweep{i}", T=T, H=H, V=V, Vu=Vu, x_std=1.0,
        w_std=float(rng.choice([0.5, 1.0, 2.0])) / math.sqrt(H), pad_std=float(rng.choice([1.0, 30.0])),
        head_fp32=bool(rng.random() < 0.25), softcap=float(rng.choice([0.0, 0.0, 5.0, 30.0])),
        reduction=str(rng.choice(["sum", "mean"])), ignore="runs" if rng.random() < 0.25 else "uniform",
        ignore_frac=ignore_frac, normalise_by_count=bool(rng.random() < 0.2))
    opts = dict(dw_tile=[None, 256, 384][int(rng.integers(0, 3 if H >= 384 else 2))],
                fp32_head_direct=w.head_fp32 and bool(rng.random() < 0.5),
                head_staged=bool(rng.random() < 0.5))
    return w, opts


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_small_problem(i):
    w, opts = draw_case(i)
    say(f"sweep {i}: T={w.T} H={w.H} V={w.V} Vu={w.Vu} c={w.softcap} {w.reduction} ignore={w.ignore}:"
        f"{w.ignore_frac} fp32={w.head_fp32} count={w.normalise_by_count} {opts}")
    inp = make_inputs(w)
    if inp["num_label_tokens"] == 0:
        # Every position ignored with the normaliser taken from the count: a
        # normaliser of 0 is refused before anything is launched.
        with pytest.raises(ValueError, match="invalid argument"):
            run_hip(inp, **opts)
        return
    res = run_hip(inp, **opts)
    assert res["status"] == 0
    check_full(inp, res, label=f"sweep{i}")
