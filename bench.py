#!/usr/bin/env python3
"""Fused linear cross-entropy forward + backward throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 2]

One step is flce_forward followed by flce_backward (every kernel of the hot
path) over one batch of synthetic inputs already resident in HBM.  Prints
one JSON line: tokens/s, the % of the bf16 dense MFMA peak that the credited
work (8 Tv Vu H flops: projection, recompute, dX and dW) reaches, a roofline
entry for the dominant kernel from HIP events recorded around each of its
launches inside the timed region (the trace records only that kernel's
launches there; the per-kernel breakdown comes from the last warmup steps),
and the CPU oracle timed on a bounded slice of the same workload.  The same
steps without any trace are timed afterwards and reported beside it;
--graph also times one step captured as a HIP graph.

    python bench.py --path chunked_ce [--ce-workload ce2]

times the cross-entropy over given logits (chunked_ce_forward +
chunked_ce_backward) instead, against the HBM roofline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense bf16 MFMA (MI355X published)
MI355X_CLOCK_GHZ = 2.4      # published peak engine clock
FLOP_PER_CLK_CU = 4096      # dense bf16 MFMA, per compute unit
METRIC = "fused linear-CE fwd+bwd tokens/sec on 1 MI355X; % of bf16 MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the HIP sources; HBM byte counts measured on other sources are stale."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lm_head_cross_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(inp, n_tokens):
    """Time the oracle (fwd + bwd, full vocabulary) on the first n_tokens
    positions of the workload; returns tokens/s, what was run, the CPU, and
    the whole workload's time extrapolated from the sample (the oracle's work
    is linear in the positions: each one's logits, softmax and gradient rows,
    and its share of dW)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"),
                      default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    X = oracle.to_f64(inp["hidden"][:n_tokens].cpu())
    W = oracle.head_values(inp["weight"].cpu())
    y = inp["labels"][:n_tokens].cpu().numpy()
    p = oracle.Problem(inp["unpadded_vocab"], inp["softcap"], inp["ignore_index"], inp["reduction"],
                       inp["num_label_tokens"])
    t0 = time.perf_counter()
    oracle.forward(X, W, y, p, row_block=256)
    oracle.backward(X, W, y, p, row_block=256)
    dt = time.perf_counter() - t0
    T = inp["hidden"].shape[0]
    return {
        "value": n_tokens / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"first {n_tokens} positions of the workload, fwd+bwd over the full vocabulary "
                  f"(fp64 numpy, {dt:.1f} s)",
        "cpu_model": cpu_model(),
        "logical_cpus": os.cpu_count(),
        "extrapolated_full_workload_s": round(dt * T / n_tokens, 1),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--cpu-tokens", type=int, default=3072)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, copy this many MiB once (a plain copy kernel of known size, "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch of the dominant kernel, from rocprofv3 counters")
    ap.add_argument("--path", choices=("flce", "chunked_ce"), default="flce",
                    help="flce: fused linear cross-entropy (the default workload); chunked_ce: cross-entropy "
                         "over given logits")
    ap.add_argument("--ce-workload", default="ce2", help="logits-input workload for --path chunked_ce")
    ap.add_argument("--graph", action="store_true",
                    help="also time one step captured as a HIP graph and replayed (an extra field; value stays "
                         "the eager rate)")
    ap.add_argument("--fp32-head-direct", action="store_true",
                    help="hand an fp32 head to the calls as fp32 (each call rounds and stages it, inside the "
                         "timed region) instead of rounding it once before timing")
    ap.add_argument("--round-head-on-load", action="store_true",
                    help="with --fp32-head-direct: the GEMMs round the fp32 head inside their tile loads "
                         "(FLCE_FLAG_ROUND_HEAD_ON_LOAD: no staged copy, smaller workspace, slower)")
    ap.add_argument("--dw-tile", type=int, choices=(256, 384), default=None,
                    help="fix the tile of the backward's dW contraction (FLCE_FLAG_DW_TILE_256 / _384); by "
                         "default the library picks it")
    ap.add_argument("--restage-head", action="store_true",
                    help="with --fp32-head-direct: the backward stages the head again instead of reusing the "
                         "forward's staged copy in the same workspace (FLCE_FLAG_HEAD_STAGED)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the fused linear cross-entropy path is built and timed on a "
              "single MI355X; runs on more than one GPU are not supported.", file=sys.stderr)
        sys.exit(2)

    if args.path == "chunked_ce":
        return bench_chunked_ce(args)

    import torch

    import lm_head_cross_amd as L
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"workload {w.key}: {w.name}")
    inp = make_inputs(w, device="cuda:0", argmax_device="cuda:0")
    X, y = inp["hidden"], inp["labels"]
    W = inp["weight"]
    direct = args.fp32_head_direct and W.dtype == torch.float32
    if W.dtype == torch.float32 and not direct:
        W = L.flce_round_to_bf16(W)
    T, H, V, Vu = w.T, w.H, w.V, w.Vu
    Tv = inp["n_valid"]
    p = L.make_problem(T, H, V, Vu, w.softcap, inp["ignore_index"], w.reduction, inp["num_label_tokens"],
                       W.dtype, round_head_on_load=direct and args.round_head_on_load, dw_tile=args.dw_tile,
                       head_staged=not args.restage_head)
    ws = L.alloc_workspace(p, dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    g = torch.ones((), dtype=torch.float32, device=dev)
    dX = torch.empty_like(X)
    dW = torch.empty((V, H), dtype=torch.float32, device=dev)

    def step():
        L.flce_forward(p, X, W, y, loss, lse, workspace=ws)
        L.flce_backward(p, X, W, y, lse, g, dX, dW, workspace=ws)

    # Warmup: the last (up to) three warmup steps run with the library's
    # launch trace on for every kind, for the per-kernel breakdown (logged)
    # and the dominant kernel kind.
    n_prof = min(args.warmup, 3)
    for _ in range(args.warmup - n_prof):
        step()
    torch.cuda.synchronize()
    full = L.LaunchTrace(capacity=max(64, 64 * n_prof)).start()
    for _ in range(n_prof):
        step()
    torch.cuda.synchronize()
    full.stop()

    # The library prices a contraction launch at 2*T*rows*H; only the Tv
    # valid tokens are work the method does, so rescale to 2*Tv*rows*H.
    def by_kind(records):
        kinds = {}
        for kind, kms, fl in records:
            k = kinds.setdefault(kind, {"launches": 0, "ms": 0.0, "flops": 0.0})
            k["launches"] += 1
            k["ms"] += kms
            k["flops"] += fl * Tv / T
        return kinds

    def show(kinds, n_steps):
        for name, k in sorted(kinds.items(), key=lambda kv: -kv[1]["ms"]):
            tf = k["flops"] / (k["ms"] * 1e-3) / 1e12 if k["flops"] else 0.0
            log(f"  {name:12s} launches={k['launches']:5d} total={k['ms'] / n_steps:8.3f} ms/step "
                f"avg={k['ms'] / k['launches'] * 1e3:9.1f} us" + (f"  {tf:7.1f} TFLOP/s (algorithmic)" if tf else ""))

    dom_name = None
    if n_prof:
        kinds = by_kind(full.records())
        show(kinds, n_prof)
        dom_name = max(kinds.items(), key=lambda kv: kv[1]["ms"])[0]

    # The timed region: the launch trace records the dominant kind's launches
    # (an event pair around each, on its stream), and events mark each step's
    # start, the boundary between its forward and backward, and its end, all
    # on torch's current stream, which is the stream the library launches on.
    trace = L.LaunchTrace(capacity=max(64, 64 * args.steps), kinds=[dom_name] if dom_name else None).start()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        ev[i][0].record()
        L.flce_forward(p, X, W, y, loss, lse, workspace=ws)
        ev[i][1].record()
        L.flce_backward(p, X, W, y, lse, g, dX, dW, workspace=ws)
        ev[i][2].record()
    e1.record()
    torch.cuda.synchronize()
    trace.stop()
    ms = e0.elapsed_time(e1) / args.steps
    step_ms = sorted(a.elapsed_time(c) for a, _, c in ev)
    fwd_ms = sorted(a.elapsed_time(b) for a, b, _ in ev)
    bwd_ms = sorted(b.elapsed_time(c) for _, b, c in ev)
    med = lambda v: v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
    timed = by_kind(trace.records())
    if dom_name is None:  # no warmup: every kind was traced in the timed steps
        show(timed, args.steps)
        dom_name = max(timed.items(), key=lambda kv: kv[1]["ms"])[0]
    dom = timed[dom_name]

    # The same number of steps again with no events at all (reported beside
    # the timed rate).
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    untraced_ms = e0.elapsed_time(e1) / args.steps

    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        entry = tj.get(f"workload{w.key}", {}).get(dom_name)
        if entry and tj.get("kernel_source_hash") == kernel_source_hash():
            traffic = entry.get("bytes_per_launch")
    roofline = {
        "kernel": dom_name,
        "bound": "mfma",
        "achieved": round(achieved, 1),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "avg_launch_us": round(dom["ms"] / dom["launches"] * 1e3, 1),
        "flops_per_launch": dom["flops"] / dom["launches"],
    }
    credited = 8.0 * Tv * Vu * H
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    peak_dev = n_cu * MI355X_CLOCK_GHZ * FLOP_PER_CLK_CU / 1e3
    tokens_per_s = T / (ms * 1e-3)
    pct_peak = credited / (ms * 1e-3) / (PEAK_BF16_TFLOPS * 1e12) * 100.0
    log(f"step {ms:.3f} ms  {tokens_per_s:,.0f} tokens/s  {pct_peak:.1f}% of bf16 peak "
        f"(credited {credited / 1e12:.2f} TFLOP; {pct_peak * 0.75:.1f}% on the 6 Tv Vu H model flops)  "
        f"loss={loss.item():.6g}")
    log(f"  per step: median {med(step_ms):.3f} ms, min {step_ms[0]:.3f} ms; forward {med(fwd_ms):.3f} ms, "
        f"backward {med(bwd_ms):.3f} ms (medians); {n_cu} CUs -> peak {peak_dev:.1f} TFLOP/s")
    log(f"  without the launch trace: {untraced_ms:.3f} ms per step")

    graph_ms = None
    if args.graph:
        # One step captured as a HIP graph and replayed: the same kernels
        # without per-launch host work (reported beside the eager time).
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        for _ in range(args.warmup):
            gr.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
        log(f"  graph replay: {graph_ms:.3f} ms per step")

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_tokens} tokens ...")
        cpu = cpu_baseline(inp, args.cpu_tokens)
        log(f"  oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": round(pct_peak, 2),
        "pct_of_bf16_peak_model_flops": round(pct_peak * 6.0 / 8.0, 2),
        "config": {
            "workload": w.name,
            "tokens": T, "hidden": H, "vocab": V, "unpadded_vocab": Vu, "valid_tokens": Tv,
            "softcap": w.softcap, "reduction": w.reduction, "head": str(W.dtype).replace("torch.", "")
            + (" (rounded on load)" if direct and args.round_head_on_load else ""),
            "num_label_tokens": inp["num_label_tokens"],
            "dw_tile": args.dw_tile or "library's choice",
            "backward_restages_head": bool(args.restage_head),
            "credited_tflop_per_step": round(credited / 1e12, 3),
            "model_tflop_per_step": round(6.0 * Tv * Vu * H / 1e12, 3),
            "label_tokens_per_s": round(Tv / (ms * 1e-3), 1),
        },
        "step_ms": {"median": round(med(step_ms), 4), "min": round(step_ms[0], 4),
                    "fwd_median": round(med(fwd_ms), 4), "bwd_median": round(med(bwd_ms), 4),
                    "untraced": round(untraced_ms, 4)},
        "peak_from_device": {"compute_units": n_cu, "clock_ghz": MI355X_CLOCK_GHZ,
                             "tflops": round(peak_dev, 1)},
        "roofline": roofline,
        "kernel_source_hash": kernel_source_hash(),
        "cpu_baseline": cpu,
    }
    if graph_ms is not None:
        line["graph_replay_ms_per_step"] = round(graph_ms, 4)
    print(json.dumps(line), flush=True)


def cpu_baseline_ce(inp, n_rows):
    """Time the logits-input oracle (fwd + bwd) on the first n_rows positions."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"),
                      default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    z = oracle.to_f64(inp["logits"][:n_rows].cpu())
    y = inp["labels"][:n_rows].cpu().numpy()
    m = None if inp["mask"] is None else inp["mask"][:n_rows].cpu().numpy()
    p = oracle.CEProblem(ignore_index=inp["ignore_index"], reduction=inp["reduction"],
                         num_label_tokens=inp["num_label_tokens"])
    t0 = time.perf_counter()
    oracle.ce_forward(z, y, p, mask=m)
    oracle.ce_backward(z, y, p, mask=m)
    dt = time.perf_counter() - t0
    T = inp["logits"].shape[0]
    return {"value": n_rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_rows} positions of the workload, fwd+bwd over the full vocabulary "
                      f"(fp64 numpy, {dt:.1f} s)",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "extrapolated_full_workload_s": round(dt * T / n_rows, 1)}


def bench_chunked_ce(args):
    """Cross-entropy over given logits: forward + backward per step."""
    import torch

    import lm_head_cross_amd as L
    from workloads import LOGIT_WORKLOADS, make_logit_inputs

    w = LOGIT_WORKLOADS[args.ce_workload]
    dev = torch.device("cuda:0")
    log(f"logits workload {w.key}: {w.name}")
    inp = make_logit_inputs(w, device="cuda:0")
    z, y, m = inp["logits"], inp["labels"], inp["mask"]
    T, V = z.shape
    Tv = inp["n_valid"]
    esz = z.element_size()
    p = L.make_ce_problem(T, V, z.dtype, inp["ignore_index"], w.reduction, inp["num_label_tokens"])
    ws = L.alloc_ce_workspace(p, dev)
    loss = torch.empty((), device=dev)
    lse = torch.empty(T, device=dev)
    g = torch.ones((), device=dev)
    dz = torch.empty_like(z)

    def step():
        L.chunked_ce_forward(p, z, y, loss, lse, mask=m, workspace=ws)
        L.chunked_ce_backward(p, z, y, lse, g, dz, mask=m, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    trace = L.LaunchTrace(capacity=max(64, 8 * args.steps)).start()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    trace.stop()
    ms = e0.elapsed_time(e1) / args.steps
    # Algorithmic bytes per launch: the forward reads the counted rows once;
    # the backward reads them and writes every gradient row.
    alg = {"ce_forward": Tv * V * esz + T * 8, "ce_backward": Tv * V * esz + T * V * esz + T * 8}
    kinds = {}
    for kind, kms, _ in trace.records():
        k = kinds.setdefault(kind, {"launches": 0, "ms": 0.0})
        k["launches"] += 1
        k["ms"] += kms
    for name, k in sorted(kinds.items(), key=lambda kv: -kv[1]["ms"]):
        gbs = alg[name] * k["launches"] / (k["ms"] * 1e-3) / 1e9 if name in alg else 0.0
        log(f"  {name:12s} launches={k['launches']:5d} total={k['ms'] / args.steps:8.3f} ms/step "
            f"avg={k['ms'] / k['launches'] * 1e3:9.1f} us" + (f"  {gbs:7.1f} GB/s (algorithmic)" if gbs else ""))
    dom_name, dom = max(((n, k) for n, k in kinds.items() if n in alg), key=lambda kv: kv[1]["ms"])
    achieved = alg[dom_name] * dom["launches"] / (dom["ms"] * 1e-3) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        entry = tj.get(w.key, {}).get(dom_name)
        if entry and tj.get("kernel_source_hash") == kernel_source_hash():
            traffic = entry.get("bytes_per_launch")
    step_bytes = alg["ce_forward"] + alg["ce_backward"]
    log(f"step {ms:.3f} ms  {T / (ms * 1e-3):,.0f} tokens/s  {step_bytes / (ms * 1e-3) / 1e9:.0f} GB/s "
        f"algorithmic ({step_bytes / (ms * 1e-3) / 8e12 * 100:.1f}% of HBM peak)  loss={loss.item():.6g}")
    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")
        del src, dst
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_ce(inp, 256)
        log(f"  oracle {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")
    line = {
        "metric": "chunked CE (logits input) fwd+bwd tokens/sec on 1 MI355X; % of HBM peak",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float32: "fp32"}[z.dtype],
        "data": "synthetic",
        "pct_of_hbm_peak": round(step_bytes / (ms * 1e-3) / 8e12 * 100, 2),
        "config": {"workload": w.name, "tokens": T, "vocab": V, "valid_tokens": Tv, "reduction": w.reduction,
                   "mask": m is not None, "algorithmic_gb_per_step": round(step_bytes / 1e9, 3)},
        "roofline": {"kernel": dom_name, "bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(achieved / 8000.0, 4), "traffic": traffic,
                     "avg_launch_us": round(dom["ms"] / dom["launches"] * 1e3, 1),
                     "bytes_per_launch": alg[dom_name]},
        "kernel_source_hash": kernel_source_hash(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
