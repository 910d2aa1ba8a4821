#!/usr/bin/env python3
"""Benchmark of the Muon / Newton-Schulz optimizer step on one MI355X.

A step is one muon_step call over a workload's matrices (momentum, normalisation, T
Newton-Schulz iterations, NorMuon and the weight update), inputs resident in HBM.
Prints one JSON line: NS algorithmic TFLOP/s over the whole step, step ms, the dominant
kernel's roofline (from hipEvents the library records around its launches during the timed
steps), a per-kernel breakdown, and the fp64 oracle timed on a bounded sample on the host.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config {1..7}] [--kind standard|gram]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks (dense MFMA and HBM3E)
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--kind", choices=["standard", "gram"], default=None,
                    help="override the workload's Newton-Schulz variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the oracle sample")
    ap.add_argument("--graph", action="store_true",
                    help="(default) also time the step captured once in a HIP graph and replayed")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP graph replay timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def build_inputs(wl, torch, np, synthetic, dev):
    """The workload's matrices, resident on `dev`: seeded synthetic gradients, zero weights,
    momenta and second-moment vectors."""
    W, M, G, V = [], [], [], []
    for idx, rows, cols in wl.matrices():
        g = synthetic.gradient(wl.dist, rows, cols, wl.storage, wl.index, 0, idx)
        if wl.storage == "bf16":
            G.append(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).to(dev))
            W.append(torch.zeros(rows, cols, dtype=torch.bfloat16, device=dev))
        else:
            G.append(torch.from_numpy(g).to(dev))
            W.append(torch.zeros(rows, cols, dtype=torch.float32, device=dev))
        M.append(torch.zeros(rows, cols, dtype=torch.float32, device=dev))
        V.append(torch.zeros(rows, dtype=torch.float32, device=dev))
    return W, M, G, V


GEMM_SOURCES = [os.path.join(ROOT, "muon_newton_schulz_amd", "csrc", f)
                for f in ("gemm.hip", "gemm_epilogue.inc")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(paths) -> str:
    """sha256[:16] over the concatenated GEMM sources with // comments and whitespace
    removed: it changes when the kernel code does, not when its comments do."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            for line in f:
                code = re.sub(r"\s+", "", re.sub(r"//.*", "", line))
                if code:
                    h.update(code.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when
    there is none for this kernel and workload or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get("kernels", {}).get(f"{workload}::{kernel}")
    if not ent or t.get("gemm_source_sha256_16") != source_digest(GEMM_SOURCES):
        return None
    return ent.get("bytes_per_launch")


def calibrate_copy():
    """A plain elementwise copy kernel of known size (out = in + 0 over 2^28 float32):
    reads and writes exactly 1 GiB per launch, 3 launches."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.add(src, 0.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise copy kernel", "bytes_read_per_launch": 4 * n,
                      "bytes_written_per_launch": 4 * n, "launches": 3}), flush=True)


def cpu_baseline(wl, kind, budget_s):
    """The fp64 oracle as it stands, timed on a bounded sample of the workload: the full
    Newton-Schulz orthogonalisation of the workload's matrices in order (starting over after
    the last), as many as fit the budget (at least the first; only its first iteration when
    even one full orthogonalisation would overrun the budget). Returns the oracle's algorithmic TFLOP/s (the same FLOP
    accounting as the GPU value)."""
    import numpy as np
    import oracle
    import synthetic
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    coeffs = wl.coeff_table()
    restarts = (wl.restart_before or (3,)) if kind == "gram" else ()

    def operand(idx, rows, cols):
        if wl.row_fraction < 1.0:
            rows = oracle.rows_for_fraction(wl.row_fraction, rows)
        g = synthetic.gradient(wl.dist, rows, cols, wl.storage, wl.index, 0, idx)
        return synthetic.decode(g, wl.storage).astype(np.float64)

    def run(x, cs):
        c = oracle.FlopCounter()
        t0 = time.perf_counter()
        oracle.orthogonalize(x, cs, kind, restarts if len(cs) == len(coeffs) else (), c)
        return c.algorithmic, time.perf_counter() - t0

    mats = wl.matrices()
    idx, rows, cols = mats[0]
    x = operand(idx, rows, cols)
    flops, dt = run(x, coeffs[:1])
    if dt * len(coeffs) >= budget_s or len(coeffs) == 1:
        return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
                "kind": "oracle",
                "sample": f"{kind} NS of matrix 0 ({x.shape[0]}x{x.shape[1]}) of "
                          f"{wl.n_matrices}, 1 of {len(coeffs)} iterations, fp64 NumPy, "
                          f"{dt:.1f} s"}
    # The workload's matrices in order, starting over after the last one, until one more
    # orthogonalisation would overrun the budget.
    flops, dt, done, last = 0, 0.0, 0, 0.0
    cache = {0: x}
    while not (done and dt + last > budget_s):
        j = done % len(mats)
        if j not in cache:
            if len(cache) > 8:
                cache.pop(next(k for k in cache if k != 0))
            cache[j] = operand(*mats[j])
        f, t = run(cache[j], coeffs)
        flops, dt, done, last = flops + f, dt + t, done + 1, t
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{kind} NS ({len(coeffs)} iterations) of {done} matrices taken in order "
                      f"from the workload's {wl.n_matrices} (cycling; operand "
                      f"{x.shape[0]}x{x.shape[1]} first), fp64 NumPy, {dt:.1f} s"}


def graph_timing(mns, torch, step_args, ws, kw, warmup, steps):
    """The same step recorded once into a HIP graph (torch.cuda.CUDAGraph on the capture
    stream) and replayed: ms per replayed step."""
    W, M, G, v = step_args
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mns.muon_step(W, M, G, v, workspace=ws, stream=torch.cuda.current_stream(), **kw)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return {"ms_per_step": round(e0.elapsed_time(e1) / steps, 4), "steps": steps}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this optimizer-step library has no multi-GPU "
              "path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import muon_newton_schulz_amd as mns
    import synthetic

    wl = synthetic.WORKLOADS[args.config]
    kind = args.kind or wl.kind
    restarts = wl.restart_before if kind == "gram" else ()
    if kind == "gram" and not restarts:
        restarts = (3,)
    dev = torch.device("cuda:0")
    W, M, G, V = build_inputs(wl, torch, np, synthetic, dev)
    kw = dict(mu=wl.mu, lr=wl.lr, coeffs=wl.coeff_table(), kind=kind, restart_before=restarts,
              normuon=wl.normuon, beta2=wl.beta2, eps=wl.eps, row_fraction=wl.row_fraction)
    v_arg = V if wl.normuon else None
    ws = torch.empty(mns.step_workspace_size(W, M, G, v_arg, **kw), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        mns.muon_step(W, M, G, v_arg, workspace=ws, stream=stream, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mns.profile_begin()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    stats = mns.profile_end()
    total_ms = e0.elapsed_time(e1)
    ms_step = total_ms / args.steps

    gemm = [s for s in stats if s["flops"] > 0]
    ns_flops = sum(s["flops"] for s in gemm) / args.steps
    ns_ms = sum(s["ms"] for s in gemm) / args.steps
    dtype = "f32" if wl.storage == "f32" else "f16"
    peak = PEAK_TFLOPS[dtype]
    value = ns_flops / (ms_step * 1e-3) / 1e12

    kernels = {}
    for s in stats:
        avg_us = 1e3 * s["ms"] / max(s["launches"], 1)
        ent = {"launches": s["launches"], "avg_us": round(avg_us, 2),
               "share": round(s["ms"] / max(total_ms, 1e-9), 4)}
        if s["flops"] > 0:
            tf = s["flops"] / (s["ms"] * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), frac=round(tf / peak, 4))
        else:
            gbs = s["bytes"] / (s["ms"] * 1e-3) / 1e9
            ent.update(gbs=round(gbs, 1), frac=round(gbs / PEAK_HBM_GBS, 4))
        kernels[s["name"]] = ent

    dom = max(stats, key=lambda s: s["ms"])
    if dom["flops"] > 0:
        ach = dom["flops"] / dom["launches"] / (dom["ms"] / dom["launches"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom["name"], "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "traffic": measured_traffic(dom["name"], f"config{args.config}-{kind}")}
    else:
        ach = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom["name"], "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(dom["name"], f"config{args.config}-{kind}")}

    graph = None
    if not args.no_graph:
        graph = graph_timing(mns, torch, step_args=(W, M, G, v_arg), ws=ws, kw=kw,
                             warmup=args.warmup, steps=args.steps)
        graph["eager_ms_per_step"] = round(ms_step, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, kind, args.cpu_seconds)

    out = {
        "metric": "NS orthogonalization TFLOP/s + Muon step ms per shape; % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.storage == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "ns": kind, "T": wl.T, "normuon": wl.normuon,
                   "row_fraction": wl.row_fraction, "matrices": wl.n_matrices,
                   "storage": wl.storage},
        "ns_gemm_ms_per_step": round(ns_ms, 4),
        "ns_gemm_tflops": round(ns_flops / (ns_ms * 1e-3) / 1e12, 1) if ns_ms > 0 else None,
        "ns_flops_per_step": ns_flops,
        "mfma_frac_step": round(value / peak, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "graph": graph,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
