"""Seeded synthetic workloads for fused linear cross-entropy.

This module only draws inputs: hidden states, head weights and labels with
the shapes and value distributions of the five named workloads.  It holds no
part of the loss arithmetic, and both the HIP path's tests and the CPU oracle
read their inputs from here.

Random numbers come from numpy's PCG64 generator.  A tensor is filled in a
fixed number of row blocks, each with its own child stream spawned from one
``SeedSequence``, so the values do not depend on how many threads fill them.
Samples are drawn in float32 and rounded to bfloat16 by torch's
round-to-nearest-even cast.

Workloads (T tokens, H hidden, V head rows of which Vu are usable):

1. tiny: T=64, H=128, V=Vu=1000, X~N(0,1), W~N(0,0.02), 10% ignored.
2. llama3-8b head: T=4096, H=4096, V=Vu=128256, W~N(0,1/sqrt(H)), 5% ignored.
3. softcapped padded head: T=8192, H=3072, V=262144, Vu=256000, head given
   in fp32, pad rows drawn at a much larger scale, c=30, 5% ignored.
4. sparse-label packed batch: T=16384, H=5120, V=Vu=152064, about half the
   labels ignored in contiguous runs of 64..512, loss divided by the supplied
   label-token count.
5. long peaked head: T=65536, H=8192, V=Vu=128256, W~N(0,4/sqrt(H)), labels
   70% the row's argmax logit and 30% uniform, 2% ignored, c=30.

The N(0, s) notation takes s as the standard deviation.

Cross-entropy over given logits (LOGIT_WORKLOADS; the chunked CE page gives
no shapes, so these take the shapes above, with the logits drawn directly):

ce1. tiny: T=64, V=1000, fp32 logits ~N(0,1), 10% ignored (rows of 4000 B,
     not 16-byte multiples).
ce2. llama3-8b head: T=4096, V=128256, bf16 logits ~N(0,2), 5% ignored.
ce3. masked fp32: T=2048, V=256000, fp32 logits ~N(0,2); 5% of positions
     dropped by an int32 mask whose labels there are out of range; mean,
     divided by the supplied count of kept positions.
ce4. packed peaked batch: T=16384, V=152064, bf16 logits ~N(0,3) with the
     label's logit raised by 12 at 70% of positions; half the positions
     ignored in runs of 64..512; mean over the counted positions.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

IGNORE_INDEX = -100
_BLOCKS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, distributions and loss knobs of one synthetic workload."""

    key: int
    name: str
    T: int
    H: int
    V: int
    Vu: int
    x_std: float
    w_std: float
    pad_std: float = 1.0
    head_fp32: bool = False
    softcap: float = 0.0
    reduction: str = "sum"
    ignore: str = "uniform"          # "uniform" | "runs"
    ignore_frac: float = 0.0
    labels: str = "uniform"          # "uniform" | "argmax70"
    normalise_by_count: bool = False  # pass num_label_tokens = number of valid labels

    @property
    def seed(self) -> int:
        return 1000 + self.key


WORKLOADS = {
    1: Workload(1, "tiny T=64 H=128 V=1000", 64, 128, 1000, 1000, 1.0, 0.02,
                ignore_frac=0.10),
    2: Workload(2, "llama3-8b head T=4096 H=4096 V=128256", 4096, 4096, 128256, 128256,
                1.0, 1.0 / math.sqrt(4096), ignore_frac=0.05),
    3: Workload(3, "softcapped padded head T=8192 H=3072 V=262144 Vu=256000", 8192, 3072,
                262144, 256000, 1.0, 1.0 / math.sqrt(3072), pad_std=1.0, head_fp32=True,
                softcap=30.0, ignore_frac=0.05),
    4: Workload(4, "sparse-label packed batch T=16384 H=5120 V=152064", 16384, 5120, 152064,
                152064, 1.0, 1.0 / math.sqrt(5120), ignore="runs", reduction="mean",
                normalise_by_count=True),
    5: Workload(5, "long peaked head T=65536 H=8192 V=128256", 65536, 8192, 128256, 128256,
                1.0, 4.0 / math.sqrt(8192), softcap=30.0, ignore_frac=0.02,
                labels="argmax70"),
}


def _normal_f32(shape, seed_seq: np.random.SeedSequence, scale: float) -> np.ndarray:
    """Fill a float32 array with N(0, scale) in _BLOCKS fixed row blocks."""
    rows = shape[0]
    out = np.empty(shape, np.float32)
    nblk = min(_BLOCKS, rows)
    children = seed_seq.spawn(nblk)
    bounds = [(rows * i) // nblk for i in range(nblk + 1)]

    def fill(i):
        g = np.random.Generator(np.random.PCG64(children[i]))
        blk = out[bounds[i]:bounds[i + 1]]
        g.standard_normal(out=blk, dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def _ignore_mask(w: Workload, rng: np.random.Generator) -> np.ndarray:
    """Boolean [T] mask of ignored positions."""
    T = w.T
    mask = np.zeros(T, dtype=bool)
    if w.ignore == "uniform":
        n = int(round(w.ignore_frac * T))
        mask[rng.permutation(T)[:n]] = True
    elif w.ignore == "runs":
        # Alternating runs of valid / ignored positions, each of length
        # uniform in [64, 512]; the first run's state is a fair coin.
        state = bool(rng.integers(0, 2))
        t = 0
        while t < T:
            n = int(rng.integers(64, 513))
            mask[t:t + n] = state
            state = not state
            t += n
    else:
        raise ValueError(f"unknown ignore pattern {w.ignore!r}")
    return mask


def _argmax_labels(X: torch.Tensor, W: torch.Tensor, Vu: int, device) -> np.ndarray:
    """Index of each row's largest head logit over the first Vu rows.

    Computed with torch float32 matmuls in token chunks on ``device``; only
    used to synthesise peaked labels, so its rounding does not matter.
    """
    dev = torch.device(device)
    Wd = W[:Vu].to(dev).float()
    out = []
    chunk = 4096 if dev.type == "cuda" else 256
    for t0 in range(0, X.shape[0], chunk):
        xs = X[t0:t0 + chunk].to(dev).float()
        out.append(torch.argmax(xs @ Wd.T, dim=1).cpu())
    del Wd
    return torch.cat(out).numpy().astype(np.int64)


def draw_hidden_and_head(w: Workload):
    """Hidden states (bf16 [T,H]) and head (bf16, or fp32 when the workload
    hands it over in fp32, [V,H]) of one workload, on the CPU."""
    sx, sw, _ = np.random.SeedSequence(w.seed).spawn(3)
    X = torch.from_numpy(_normal_f32((w.T, w.H), sx, w.x_std)).to(torch.bfloat16)
    Wf = _normal_f32((w.V, w.H), sw, w.w_std)
    if w.V > w.Vu:
        # Padding rows: drawn at their own scale so that letting them into the
        # softmax would visibly change every result.
        Wf[w.Vu:] *= np.float32(w.pad_std / w.w_std)
    Wt = torch.from_numpy(Wf)
    if not w.head_fp32:
        Wt = Wt.to(torch.bfloat16)
    return X, Wt


def make_inputs(key_or_workload, device="cpu", argmax_device=None):
    """Draw one workload's inputs.

    Returns a dict with ``hidden`` (bf16 [T,H]), ``weight`` (bf16 [V,H], or
    fp32 when the workload hands the head over in fp32), ``labels`` (int64 [T])
    and the workload's loss knobs.  Tensors are placed on ``device``.
    ``argmax_device`` is where peaked labels are searched (default: ``device``).
    """
    w = key_or_workload if isinstance(key_or_workload, Workload) else WORKLOADS[key_or_workload]
    X, Wt = draw_hidden_and_head(w)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed).spawn(3)[2]))

    ignored = _ignore_mask(w, rng)
    labels = rng.integers(0, w.Vu, size=w.T, dtype=np.int64)
    if w.labels == "argmax70":
        take = rng.random(w.T) < 0.7
        Wb = Wt if Wt.dtype == torch.bfloat16 else Wt.to(torch.bfloat16)
        am = _argmax_labels(X, Wb, w.Vu, argmax_device or device)
        labels = np.where(take, am, labels)
    elif w.labels != "uniform":
        raise ValueError(f"unknown label scheme {w.labels!r}")
    labels[ignored] = IGNORE_INDEX
    n_valid = int((~ignored).sum())

    dev = torch.device(device)
    return {
        "workload": w,
        "hidden": X.to(dev),
        "weight": Wt.to(dev),
        "labels": torch.from_numpy(labels).to(dev),
        "unpadded_vocab": w.Vu,
        "softcap": w.softcap,
        "ignore_index": IGNORE_INDEX,
        "reduction": w.reduction,
        "num_label_tokens": n_valid if w.normalise_by_count else None,
        "n_valid": n_valid,
    }


def sample_rows(key_or_workload, labels: np.ndarray, n_tokens=512, n_vocab=512, tile=256):
    """Seeded check subsets for a large workload.

    Tokens: t=0, t=T-1, positions at tile edges, then uniform picks (ignored
    positions included).  Vocab rows: 0, Vu-1, tile edges, the labels of 64
    checked tokens, then uniform picks.  Sorted, without duplicates.
    """
    w = key_or_workload if isinstance(key_or_workload, Workload) else WORKLOADS[key_or_workload]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed + 7)))
    T, Vu = w.T, w.Vu
    tok = {0, T - 1}
    for e in range(tile, T, tile * max(1, T // (tile * 16))):
        tok.update({e - 1, e})
    while len(tok) < min(n_tokens, T):
        tok.add(int(rng.integers(0, T)))
    tok = np.array(sorted(tok), dtype=np.int64)

    voc = {0, Vu - 1}
    for e in range(tile, Vu, tile * max(1, Vu // (tile * 16))):
        voc.update({e - 1, e})
    lab = labels[tok]
    lab = lab[(lab >= 0) & (lab < Vu)]
    voc.update(int(v) for v in lab[:64])
    while len(voc) < min(n_vocab, Vu):
        voc.add(int(rng.integers(0, Vu)))
    voc = np.array(sorted(voc), dtype=np.int64)
    return tok, voc


# ---------------------------------------------------------------------------
# Cross-entropy over given logits
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class LogitsWorkload:
    """Shape and value distributions of one logits-input workload."""

    key: str
    name: str
    T: int
    V: int
    dtype: str             # "bf16" | "fp32"
    std: float
    ignore: str = "uniform"
    ignore_frac: float = 0.0
    reduction: str = "sum"
    normalise_by_count: bool = False
    use_mask: bool = False  # drop positions through an int32 mask instead of ignore_index
    peak: float = 0.0       # added to the label's logit at 70% of positions

    @property
    def seed(self) -> int:
        return 2000 + int(self.key[2:])


LOGIT_WORKLOADS = {
    "ce1": LogitsWorkload("ce1", "tiny logits T=64 V=1000 fp32", 64, 1000, "fp32", 1.0, ignore_frac=0.10),
    "ce2": LogitsWorkload("ce2", "llama3-8b logits T=4096 V=128256 bf16", 4096, 128256, "bf16", 2.0,
                          ignore_frac=0.05),
    "ce3": LogitsWorkload("ce3", "masked fp32 logits T=2048 V=256000", 2048, 256000, "fp32", 2.0, ignore_frac=0.05,
                          reduction="mean", normalise_by_count=True, use_mask=True),
    "ce4": LogitsWorkload("ce4", "packed peaked logits T=16384 V=152064 bf16", 16384, 152064, "bf16", 3.0,
                          ignore="runs", reduction="mean", peak=12.0),
}


def make_logit_inputs(key_or_workload, device="cpu"):
    """Draw one logits-input workload.

    Returns ``logits`` ([T,V], bf16 or fp32), ``labels`` (int64 [T]), ``mask``
    (int32 [T] or None) and the loss knobs, on ``device``.  With a mask, the
    dropped positions carry labels outside [0, V) that the mask must hide.
    """
    w = key_or_workload if isinstance(key_or_workload, LogitsWorkload) else LOGIT_WORKLOADS[key_or_workload]
    sz, sl = np.random.SeedSequence(w.seed).spawn(2)
    Z = _normal_f32((w.T, w.V), sz, w.std)
    rng = np.random.Generator(np.random.PCG64(sl))
    shape_only = Workload(key=0, name=w.name, T=w.T, H=1, V=w.V, Vu=w.V, x_std=1.0, w_std=1.0, ignore=w.ignore,
                          ignore_frac=w.ignore_frac)
    dropped = _ignore_mask(shape_only, rng)
    labels = rng.integers(0, w.V, size=w.T, dtype=np.int64)
    if w.peak:
        boost = np.nonzero(rng.random(w.T) < 0.7)[0]
        Z[boost, labels[boost]] += np.float32(w.peak)
    mask = None
    if w.use_mask:
        mask = (~dropped).astype(np.int32)
        labels[dropped] = w.V + rng.integers(0, 1000, size=int(dropped.sum()))
    else:
        labels[dropped] = IGNORE_INDEX
    n_valid = int((~dropped).sum())
    logits = torch.from_numpy(Z)
    if w.dtype == "bf16":
        logits = logits.to(torch.bfloat16)
    del Z
    dev = torch.device(device)
    return {
        "workload": w,
        "logits": logits.to(dev),
        "labels": torch.from_numpy(labels).to(dev),
        "mask": None if mask is None else torch.from_numpy(mask).to(dev),
        "ignore_index": IGNORE_INDEX,
        "reduction": w.reduction,
        "num_label_tokens": n_valid if w.normalise_by_count else None,
        "n_valid": n_valid,
    }


def sample_logit_rows(key_or_workload, counted: np.ndarray, n_rows=512, n_ignored=64):
    """Seeded positions for sampled gradient checks: 0 and T-1, at least
    ``n_rows`` counted positions (all if fewer), and up to ``n_ignored``
    ignored ones (whose gradient rows must be zero)."""
    w = key_or_workload if isinstance(key_or_workload, LogitsWorkload) else LOGIT_WORKLOADS[key_or_workload]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed + 7)))
    on = np.nonzero(counted)[0]
    off = np.nonzero(~counted)[0]
    rows = {0, w.T - 1}
    rows.update(int(v) for v in rng.choice(on, size=min(n_rows, len(on)), replace=False))
    if len(off):
        rows.update(int(v) for v in rng.choice(off, size=min(n_ignored, len(off)), replace=False))
    return np.array(sorted(rows), dtype=np.int64)
