"""Write the CPU oracle's per-token log-sum-exp for the large workloads.

The stored values are label independent (lse_t = log sum_{v<Vu} exp z'_tv),
so they hold for every token of workloads 2-5 whatever the labels are.  GPU
parity tests read them to check the total loss and dW rows without a
multi-minute fp64 pass.  This script calls only ``oracle`` (and the seeded
input generators); run it from the repository root:

    python tests/golden/make_oracle_lse.py 2 3 4 5
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import WORKLOADS, draw_hidden_and_head  # noqa: E402


def lse_path(key: int) -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), f"oracle_lse_w{key}.npy")


def main(keys):
    for k in keys:
        w = WORKLOADS[k]
        t0 = time.time()
        # lse does not depend on the labels: draw hidden states and head only.
        X, Wt = draw_hidden_and_head(w)
        Xv = oracle.to_f64(X)
        Wv = oracle.head_values(Wt)[: w.Vu]
        p = oracle.Problem(w.Vu, w.softcap)
        lse = oracle.token_lse(Xv, Wv, p, row_block=512)
        np.save(lse_path(k), lse)
        print(f"workload {k}: T={w.T} lse written in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [2, 3, 4, 5])
