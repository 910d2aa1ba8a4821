"""bench.py on a GPU: the one JSON line it prints carries the fields the measurement contract
asks for, with values that agree with each other (a short run on the small float32 workload, and
on the 4 x 4096^2 workload with the 4096x16384 gate and the Gram comparison)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    print("bench.py", *args, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                       text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _common(d, steps, warmup):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
              "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["data"] == "synthetic"
    # value = NS algorithmic FLOPs per step over the step time
    assert abs(d["value"] - d["ns_flops_per_step"] / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # the roofline kernel is the one that takes the most time
    kern = d["kernels"][roof["kernel"]]
    assert all(kern["share"] >= v["share"] for v in d["kernels"].values())


def test_bench_line_small_float32():
    d = _run("--workload", "1", "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-graph")
    _common(d, 3, 1)
    assert d["dtype"] == "f32" and d["cpu_baseline"] is None
    roof = d["roofline"]
    assert roof["peak"] == (157.3 if roof["bound"] == "mfma" else 8000.0)


def test_bench_line_with_gate_and_gram():
    d = _run("--workload", "2", "--steps", "3", "--warmup", "1", "--cpu-seconds", "3")
    _common(d, 3, 1)
    assert d["dtype"] == "f16" and d["roofline"]["peak"] == 2500.0
    gate = d["ns_gate_4096x16384"]
    assert gate["ns"] == "standard" and 0 < gate["ns_gemm_frac"] < 1
    gram = d["gram_ns_same_matrices"]
    assert gram["ms_per_step"] > 0 and gram["step_speedup_vs_standard"] > 0
    assert d["graph"]["ms_per_step"] > 0
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["os_cpu_count"] >= 1
    assert "sys_clock_mhz" in d["gpu_clocks"]
    flushed = d["hbm_kernels_cache_flushed"]["kernels"]
    assert "momentum" in flushed and 0 < flushed["momentum"]["frac"] < 1
    # the MFMA-only ceiling: below the published peak's reach, above what the GEMMs achieve
    # per launch, and the fractions of it consistent with the rates they divide
    ceil = d["mfma_ceiling"]
    assert 0 < ceil["tflops"] <= 1.05 * 2500.0
    assert ceil["zero_operands"]["checksum"] == 0.0
    assert abs(d["roofline"]["frac_of_sustained_mfma"] - d["roofline"]["achieved"] / ceil["tflops"]) < 1e-3
    assert abs(gate["ns_gemm_frac_of_sustained_mfma"] - gate["ns_gemm_tflops"] / ceil["tflops"]) < 1e-3
