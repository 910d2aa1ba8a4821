#!/usr/bin/env python3
"""Benchmark of the Muon / Newton-Schulz optimizer step on one MI355X.

A step is one muon_step call over a workload's matrices (momentum, normalisation, T
Newton-Schulz iterations, NorMuon and the weight update), inputs resident in HBM. The
default workload is the largest: the 196-matrix layer set of a 3B-like transformer
(28 x {4 x 3072^2, 2 x 3072x8192, 1 x 8192x3072} bf16, NorMuon). Prints one JSON line:

  * value: NS algorithmic TFLOP/s over the whole step (symmetric products priced at half the
    dense 2MNK); ms_per_step over K timed steps as a caller runs them (the library's per-launch
    events off; ms_per_step_instrumented is the same K steps with them on, the run the
    roofline's per-launch times come from); the dense-equivalent rate beside it;
  * roofline: the dominant kernel's algorithmic FLOPs per launch over its mean launch time,
    from hipEvents the library records around each of its launches during the timed steps;
  * kernels: per-kernel breakdown of the timed steps;
  * hbm_kernels_cache_flushed: the elementwise / reduction kernels timed again with a 1 GiB
    buffer written before each launch (the 256 MB Infinity Cache evicted);
  * ns_gate_4096x16384: the 4096x16384 bf16 standard-NS step timed in the same process, its
    Newton-Schulz GEMM phase as a fraction of the bf16 MFMA peak;
  * gram_ns_same_matrices: the step with Gram Newton-Schulz (restart before iteration 3) on
    the same resident matrices, and its speedup over the standard-NS step;
  * gpu_clocks: the graphics and memory clocks (and socket power) read during the timed steps;
  * mfma_ceiling: the rate of an MFMA-only kernel (no memory traffic) with random and with
    zero float16 operands on this part, right after the timed work: what the matrix pipes
    sustain at the clock the power limit leaves them; the roofline and the gate are also
    given as fractions of it (beside the published peak, which stays their `peak`);
  * cpu_baseline: the fp64 oracle on a bounded sample, on the host's cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload {1..7}] [--kind standard|gram]
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
PEAK_CLOCK_MHZ = 2400.0       # the clock the published MFMA peaks are quoted at
DEFAULT_WORKLOAD = 4          # the 196-matrix layer set (the largest workload)
GATE_WORKLOAD = 3             # 4096x16384 bf16, standard NS: the MFMA gate (>= 60 % of peak)
MFMA_GATE = 0.60
HBM_GATE = 0.70
FLUSH_BYTES = 1 << 30


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", "--config", dest="workload", type=int, default=DEFAULT_WORKLOAD,
                    choices=[1, 2, 3, 4, 5, 6, 7])
    ap.add_argument("--kind", choices=["standard", "gram"], default=None,
                    help="override the workload's Newton-Schulz variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-clock budget of the oracle sample")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP graph replay timing")
    ap.add_argument("--no-gate", action="store_true",
                    help="skip the 4096x16384 standard-NS gate timing")
    ap.add_argument("--no-flush-pass", action="store_true",
                    help="skip the cache-flushed timing of the HBM kernels")
    ap.add_argument("--no-gram", action="store_true",
                    help="skip the Gram NS timing on the same matrices")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the MFMA-only ceiling probe and print its JSON")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the MFMA-only ceiling probe (kernel traces of the step alone)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args(argv)


def gradient_bits(wl, synthetic, threads: int = 8):
    """The workload's seeded gradients (stored bits), drawn on `threads` host threads (the
    generators release the GIL); the same bits as synthetic.gradient one by one."""
    from concurrent.futures import ThreadPoolExecutor
    mats = wl.matrices()

    def one(m):
        idx, rows, cols = m
        return synthetic.gradient(wl.dist, rows, cols, wl.storage, wl.index, 0, idx)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        yield from ex.map(one, mats)


def build_inputs(wl, torch, np, synthetic, dev):
    """The workload's matrices, resident on `dev`: seeded synthetic gradients, zero weights,
    momenta and second-moment vectors."""
    W, M, G, V = [], [], [], []
    for (idx, rows, cols), g in zip(wl.matrices(), gradient_bits(wl, synthetic)):
        if wl.storage == "bf16":
            G.append(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).to(dev))
            W.append(torch.zeros(rows, cols, dtype=torch.bfloat16, device=dev))
        else:
            G.append(torch.from_numpy(g).to(dev))
            W.append(torch.zeros(rows, cols, dtype=torch.float32, device=dev))
        M.append(torch.zeros(rows, cols, dtype=torch.float32, device=dev))
        V.append(torch.zeros(rows, dtype=torch.float32, device=dev))
    return W, M, G, V


def ns_shapes(wl):
    """(n, m) of the Newton-Schulz problem of every matrix: n the short side (the selected
    rows under Dion3), m the long side."""
    import math
    out = []
    for _, rows, cols in wl.matrices():
        if wl.row_fraction < 1.0:
            rows = max(1, min(rows, math.ceil(wl.row_fraction * rows)))
        out.append((min(rows, cols), max(rows, cols)))
    return out


def dense_equivalent_flops(wl) -> float:
    """FLOPs of standard NS with every product computed dense, T (4 m n^2 + 2 n^3) per matrix
    (the dense count the page's FLOP analysis starts from)."""
    return float(sum(wl.T * (4 * m * n * n + 2 * n ** 3) for n, m in ns_shapes(wl)))


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


def host_info():
    """Host CPU model, logical CPUs, and the BLAS library the oracle's NumPy uses."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = [], None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas.append({k: i.get(k) for k in ("internal_api", "version", "num_threads",
                                                    "threading_layer", "architecture")})
                threads = max(threads or 0, int(i.get("num_threads") or 0))
    except Exception:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
            "blas": blas}, threads


def cpu_baseline(wl, kind, budget_s):
    """The fp64 oracle as it stands, timed on a bounded sample of the workload: the full
    Newton-Schulz orthogonalisation of the workload's matrices in order (starting over after
    the last), as many as fit the budget (at least the first; only its first iteration when
    even one full orthogonalisation would overrun the budget). Returns the oracle's
    algorithmic TFLOP/s (the same FLOP accounting as the GPU value)."""
    import numpy as np
    import oracle
    import synthetic
    info, threads = host_info()
    threads = threads or os.cpu_count() or 1
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
                          f"{dt:.1f} s", **info}
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
                      f"{x.shape[0]}x{x.shape[1]} first), fp64 NumPy, {dt:.1f} s", **info}


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
    del g
    return {"ms_per_step": round(e0.elapsed_time(e1) / steps, 4), "steps": steps}


def kernel_table(stats, total_ms, peak):
    kernels = {}
    for s in stats:
        avg_us = 1e3 * s["ms"] / max(s["launches"], 1)
        ent = {"launches": s["launches"], "avg_us": round(avg_us, 2)}
        if total_ms:
            ent["share"] = round(s["ms"] / max(total_ms, 1e-9), 4)
        if s["flops"] > 0:
            tf = s["flops"] / (s["ms"] * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), frac=round(tf / peak, 4))
        else:
            gbs = s["bytes"] / (s["ms"] * 1e-3) / 1e9
            ent.update(gbs=round(gbs, 1), frac=round(gbs / PEAK_HBM_GBS, 4))
        kernels[s["name"]] = ent
    return kernels


class ClockSampler:
    """The GPU's graphics (SYS) and memory clocks and its socket power, read through amdsmi
    while timed work drains (the clock this part sustains under MFMA load is well below the
    2.4 GHz of the published peak). Every field is None where the library or the reading is
    unavailable."""

    _lib = None          # amdsmi, initialised once per process (shut down at exit)

    @classmethod
    def _amdsmi(cls):
        if cls._lib is None:
            import atexit
            import amdsmi
            amdsmi.amdsmi_init()
            atexit.register(amdsmi.amdsmi_shut_down)
            cls._lib = amdsmi
        return cls._lib

    def __init__(self):
        self.h = None
        self.sys, self.mem, self.power = [], [], []
        self.t0 = self.t1 = None
        try:
            amdsmi = self._amdsmi()
            hs = amdsmi.amdsmi_get_processor_handles()
            if len(hs) == 1:
                self.amdsmi, self.h = amdsmi, hs[0]
        except Exception:
            self.h = None

    def sample(self):
        if self.h is None:
            return
        now = time.perf_counter()
        self.t0 = now if self.t0 is None else self.t0
        self.t1 = now
        a = self.amdsmi
        try:
            self.sys.append(a.amdsmi_get_clock_info(self.h, a.AmdSmiClkType.SYS)["clk"])
            self.mem.append(a.amdsmi_get_clock_info(self.h, a.AmdSmiClkType.MEM)["clk"])
        except Exception:
            pass
        try:
            pw = a.amdsmi_get_power_info(self.h)
            w = pw.get("current_socket_power") or pw.get("average_socket_power")
            if isinstance(w, (int, float)):
                self.power.append(float(w))
        except Exception:
            pass

    def summary(self):
        def stats(v):
            v = [x for x in v if isinstance(x, (int, float))]
            return {"mean": round(sum(v) / len(v), 1), "min": min(v), "max": max(v)} if v else None
        # amdsmi refreshes these readings about once a second: a window much shorter than that
        # can show the values from before the work started
        window = round(self.t1 - self.t0, 3) if self.t0 is not None else None
        out = {"sys_clock_mhz": stats(self.sys), "mem_clock_mhz": stats(self.mem),
               "socket_power_w": stats(self.power), "samples": len(self.sys),
               "window_s": window, "reliable": window is not None and window >= 1.0,
               "source": "amdsmi" if self.h is not None else None}
        # context: the published dense peak assumes 2.4 GHz; the peak at the clock held here
        if out["sys_clock_mhz"]:
            out["f16_peak_tflops_at_mean_clock"] = round(
                PEAK_TFLOPS["f16"] * out["sys_clock_mhz"]["mean"] / PEAK_CLOCK_MHZ, 1)
        return out


def mfma_ceiling(torch, iters=30000, reps=24):
    """The MFMA-only probe (libmns_probe.so): `reps` launches of about 40 ms each with random
    float16 operands, then with zero operands; each rate is the median of the second half of
    its launches (after the clock has settled). The clock each ran at comes from counters
    (GRBM_GUI_ACTIVE under rocprofv3): amdsmi's readings trail a change of load by most of a
    second."""
    from muon_newton_schulz_amd import probe
    stream = torch.cuda.current_stream()
    out = {"kernel": "v_mfma_f32_32x32x16_f16 only, 4 independent accumulators per wave, "
                     "8 workgroups of 4 waves per CU, no memory traffic in the loop",
           "iters": iters, "launches": reps}
    for zero in (False, True):
        times, flops = [], 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            flops = probe.mfma_launch(iters, zero, stream)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        settled = sorted(times[reps // 2:])
        ms = settled[len(settled) // 2]
        check = probe.mfma_checksum(4096)
        key = "zero_operands" if zero else "random_operands"
        out[key] = {"tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["f16"], 4),
                    "ms_per_launch": round(ms, 3), "checksum": check}
    out["tflops"] = out["random_operands"]["tflops"]
    return out


class Workload:
    """One workload resident on the GPU, with its step arguments and workspace."""

    def __init__(self, wl, kind, torch, np, mns, synthetic, dev):
        self.wl, self.kind, self.torch, self.mns = wl, kind, torch, mns
        restarts = wl.restart_before if kind == "gram" else ()
        if kind == "gram" and not restarts:
            restarts = (3,)
        self.W, self.M, self.G, self.V = build_inputs(wl, torch, np, synthetic, dev)
        self.kw = dict(mu=wl.mu, lr=wl.lr, coeffs=wl.coeff_table(), kind=kind,
                       restart_before=restarts, normuon=wl.normuon, beta2=wl.beta2, eps=wl.eps,
                       row_fraction=wl.row_fraction)
        self.v_arg = self.V if wl.normuon else None
        self.ws = torch.empty(mns.step_workspace_size(self.W, self.M, self.G, self.v_arg, **self.kw),
                              dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()

    def step(self):
        self.mns.muon_step(self.W, self.M, self.G, self.v_arg, workspace=self.ws,
                           stream=self.stream, **self.kw)

    def run(self, steps, profile=False, flush=None, clocks=None):
        """`steps` steps between two synchronisations; returns (ms per step, kernel stats or
        None). With `profile` the library records a hipEvent pair around each launch; with
        `flush` (a device buffer) it writes over it before each HBM-bound launch; with `clocks`
        (a ClockSampler) the clocks are read every few milliseconds until the steps are done."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if profile:
            self.mns.profile_begin()
            if flush is not None:
                self.mns.profile_set_flush(flush)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(steps):
            self.step()
        e1.record(self.stream)
        if clocks is not None:
            while not e1.query():
                clocks.sample()
                time.sleep(0.005)
        torch.cuda.synchronize()
        stats = self.mns.profile_end() if profile else None
        return e0.elapsed_time(e1) / steps, stats

    def free(self):
        del self.W, self.M, self.G, self.V, self.ws


def gemm_phase(stats, steps):
    gemm = [s for s in stats if s["flops"] > 0]
    flops = sum(s["flops"] for s in gemm) / steps
    ms = sum(s["ms"] for s in gemm) / steps
    return flops, ms


def main(argv=None):
    args = parse(argv)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.mfma_ceiling:
        import torch
        print(json.dumps({"mfma_ceiling": mfma_ceiling(torch)}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this optimizer-step library has no multi-GPU "
              "path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU: no HIP device is visible", file=sys.stderr)
        sys.exit(3)

    import muon_newton_schulz_amd as mns
    import synthetic

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    wl = synthetic.WORKLOADS[args.workload]
    kind = args.kind or wl.kind
    dtype = "f32" if wl.storage == "f32" else "f16"
    peak = PEAK_TFLOPS[dtype]

    say(f"workload {args.workload}: {wl.name}; building inputs")
    t0 = time.perf_counter()
    work = Workload(wl, kind, torch, np, mns, synthetic, dev)
    say(f"inputs resident ({time.perf_counter() - t0:.1f} s); warm-up")
    work.run(args.warmup)

    # The timed steps, with the per-launch events (the roofline's source).
    say(f"timing {args.steps} steps")
    clocks = ClockSampler()
    ms_step, stats = work.run(args.steps, profile=True, clocks=clocks)
    total_ms = ms_step * args.steps
    ns_flops, ns_ms = gemm_phase(stats, args.steps)
    dense_eq = dense_equivalent_flops(wl) if kind == "standard" else None
    kernels = kernel_table(stats, total_ms, peak)

    dom = max(stats, key=lambda s: s["ms"])
    traffic_key = f"workload{args.workload}-{kind}"
    if dom["flops"] > 0:
        ach = dom["flops"] / dom["launches"] / (dom["ms"] / dom["launches"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom["name"], "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "traffic": measured_traffic(dom["name"], traffic_key),
                "flops_per_launch": dom["flops"] / dom["launches"],
                "avg_launch_us": round(1e3 * dom["ms"] / dom["launches"], 2)}
    else:
        ach = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom["name"], "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(dom["name"], traffic_key),
                "bytes_per_launch": dom["bytes"] / dom["launches"],
                "avg_launch_us": round(1e3 * dom["ms"] / dom["launches"], 2)}

    # The same steps without the per-launch events: the step time and rate reported.
    say("uninstrumented steps")
    ms_plain, _ = work.run(args.steps)
    value = ns_flops / (ms_plain * 1e-3) / 1e12

    # The HBM kernels with the Infinity Cache flushed before each launch.
    flushed = None
    if not args.no_flush_pass:
        say("cache-flushed HBM kernel timing")
        buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        n_fl = max(1, min(args.steps, 5))
        _, fstats = work.run(n_fl, profile=True, flush=buf)
        del buf
        big = [s for s in fstats if s["flops"] == 0 and s["bytes"] / s["launches"] >= 16 << 20]
        flushed = kernel_table(big, 0, peak)   # the launches that moved >= 16 MiB (flushed ones)
        flushed = {"steps": n_fl, "flush_bytes": FLUSH_BYTES, "gate": HBM_GATE, "kernels": flushed}

    # The page's Gram Newton-Schulz (Theorem 2, restart before iteration 3) on the same resident
    # matrices, for comparison with the standard NS timed above (fewer algorithmic FLOPs).
    gram = None
    if not args.no_gram and kind == "standard" and wl.n_matrices > 1:
        say("Gram NS on the same matrices")
        gkw = dict(work.kw, kind="gram", restart_before=(3,))
        gws = torch.empty(mns.step_workspace_size(work.W, work.M, work.G, work.v_arg, **gkw),
                          dtype=torch.uint8, device=dev)

        def gstep():
            mns.muon_step(work.W, work.M, work.G, work.v_arg, workspace=gws, stream=work.stream, **gkw)

        for _ in range(args.warmup):
            gstep()
        mns.profile_begin()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(work.stream)
        for _ in range(args.steps):
            gstep()
        g1.record(work.stream)
        torch.cuda.synchronize()
        gstats = mns.profile_end()
        g_ms = g0.elapsed_time(g1) / args.steps
        g_flops, g_ns_ms = gemm_phase(gstats, args.steps)
        g0.record(work.stream)
        for _ in range(args.steps):
            gstep()
        g1.record(work.stream)
        torch.cuda.synchronize()
        g_plain = g0.elapsed_time(g1) / args.steps
        gram = {"ns": "gram", "restart_before": [3], "ms_per_step": round(g_plain, 4),
                "ms_per_step_instrumented": round(g_ms, 4),
                "ns_flops_per_step": g_flops,
                "ns_gemm_tflops": round(g_flops / (g_ns_ms * 1e-3) / 1e12, 1),
                "step_speedup_vs_standard": round(ms_plain / g_plain, 3)}
        del gws

    graph = None
    if not args.no_graph:
        say("graph replay")
        graph = graph_timing(mns, torch, step_args=(work.W, work.M, work.G, work.v_arg),
                             ws=work.ws, kw=work.kw, warmup=args.warmup, steps=args.steps)
        graph["eager_ms_per_step"] = round(ms_plain, 4)
    work.free()
    del work
    torch.cuda.empty_cache()

    gate = None
    if not args.no_gate and args.workload != GATE_WORKLOAD:
        gwl = synthetic.WORKLOADS[GATE_WORKLOAD]
        say(f"gate workload: {gwl.name}, standard NS")
        gw = Workload(gwl, "standard", torch, np, mns, synthetic, dev)
        gw.run(args.warmup)
        gclocks = ClockSampler()
        g_ms, g_stats = gw.run(args.steps, profile=True, clocks=gclocks)
        g_flops, g_ns_ms = gemm_phase(g_stats, args.steps)
        g_plain, _ = gw.run(args.steps)
        gate_tf = g_flops / (g_ns_ms * 1e-3) / 1e12
        gate = {"workload": gwl.name, "ns": "standard", "ms_per_step": round(g_plain, 4),
                "ms_per_step_instrumented": round(g_ms, 4),
                "ns_gemm_ms_per_step": round(g_ns_ms, 4), "ns_gemm_tflops": round(gate_tf, 1),
                "ns_gemm_frac": round(gate_tf / PEAK_TFLOPS["f16"], 4), "gate": MFMA_GATE,
                "step_tflops": round(g_flops / (g_plain * 1e-3) / 1e12, 1),
                "dense_equivalent_tflops": round(dense_equivalent_flops(gwl) / (g_plain * 1e-3) / 1e12, 1),
                "gpu_clocks": gclocks.summary(),
                "kernels": kernel_table(g_stats, g_ms * args.steps, PEAK_TFLOPS["f16"])}
        gw.free()
        del gw
        torch.cuda.empty_cache()

    # What the matrix pipes sustain on this part right now (random operands), for reading the
    # fractions of the published peak above.
    ceiling = None
    if not args.no_mfma_ceiling:
        say("MFMA-only ceiling")
        ceiling = mfma_ceiling(torch)
        if roof["bound"] == "mfma" and dtype == "f16":
            roof["frac_of_sustained_mfma"] = round(roof["achieved"] / ceiling["tflops"], 4)
        if gate is not None:
            gate["ns_gemm_frac_of_sustained_mfma"] = round(gate["ns_gemm_tflops"] / ceiling["tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        say("oracle sample on the host")
        cpu = cpu_baseline(wl, kind, args.cpu_seconds)

    out = {
        "metric": "NS orthogonalization TFLOP/s + Muon step ms per shape; % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_plain, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "ns": kind, "T": wl.T, "normuon": wl.normuon,
                   "row_fraction": wl.row_fraction, "matrices": wl.n_matrices,
                   "storage": wl.storage},
        "ms_per_step_instrumented": round(ms_step, 4),
        "ns_gemm_ms_per_step": round(ns_ms, 4),
        "ns_gemm_tflops": round(ns_flops / (ns_ms * 1e-3) / 1e12, 1) if ns_ms > 0 else None,
        "ns_flops_per_step": ns_flops,
        "dense_equivalent_flops_per_step": dense_eq,
        "dense_equivalent_tflops": round(dense_eq / (ms_plain * 1e-3) / 1e12, 1) if dense_eq else None,
        "mfma_frac_step": round(value / peak, 4),
        "roofline": roof,
        "gpu_clocks": clocks.summary(),
        "mfma_ceiling": ceiling,
        "cpu_baseline": cpu,
        "ns_gate_4096x16384": gate,
        "gram_ns_same_matrices": gram,
        "hbm_kernels_cache_flushed": flushed,
        "graph": graph,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
