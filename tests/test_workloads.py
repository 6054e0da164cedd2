"""The seeded workload generators: determinism, shapes and label recipes."""
import numpy as np
import torch

from workloads import WORKLOADS, make_inputs, sample_rows, _ignore_mask


def test_tiny_workload_shapes_and_determinism():
    a = make_inputs(1)
    b = make_inputs(1)
    assert a["hidden"].shape == (64, 128) and a["hidden"].dtype == torch.bfloat16
    assert a["weight"].shape == (1000, 128) and a["weight"].dtype == torch.bfloat16
    assert torch.equal(a["hidden"], b["hidden"]) and torch.equal(a["weight"], b["weight"])
    assert torch.equal(a["labels"], b["labels"])
    y = a["labels"].numpy()
    assert (y == -100).sum() == 6 and a["n_valid"] == 58
    assert y[y != -100].min() >= 0 and y[y != -100].max() < 1000
    assert abs(a["weight"].float().std().item() - 0.02) < 0.002


def test_ignore_recipes():
    w3 = WORKLOADS[3]
    m = _ignore_mask(w3, np.random.default_rng(0))
    assert m.sum() == round(0.05 * w3.T)
    w4 = WORKLOADS[4]
    m = _ignore_mask(w4, np.random.default_rng(1))
    # alternating runs of 64..512 positions
    edges = np.flatnonzero(np.diff(m.astype(np.int8))) + 1
    runs = np.diff(np.concatenate([[0], edges, [w4.T]]))
    assert runs[:-1].min() >= 64 and runs.max() <= 512
    assert 0.35 < m.mean() < 0.65


def test_sample_rows_cover_edges():
    y = np.arange(4096) % 1000
    tok, voc = sample_rows(2, y)
    assert tok[0] == 0 and tok[-1] == 4095 and len(tok) >= 512
    assert voc[0] == 0 and voc[-1] == 128255 and len(voc) >= 512
    assert len(np.unique(tok)) == len(tok)
