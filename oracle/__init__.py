"""CPU oracles for fused linear cross-entropy and for cross-entropy over given
logits (test infrastructure only).

Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import this package; the product path never does.
"""
from .flce_oracle import *  # noqa: F401,F403
from .flce_oracle import Forward, Problem  # noqa: F401
from .chunked_ce_oracle import (CEProblem, apply_mask, ce_backward, ce_forward, ce_label_logits,  # noqa: F401
                                ce_loss_from_lse, ce_lse, ce_rows, check_ce_problem)
