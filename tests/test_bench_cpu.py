"""Host-side checks of bench.py: the one-GPU guard, the message without a GPU, input
construction and the counter lookup (no GPU: inputs are built on the CPU)."""
import dataclasses
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the message a machine without a GPU gets")
def test_without_a_gpu_bench_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 3
    assert "needs a GPU" in r.stderr


def test_build_inputs_matches_workload():
    wl = synthetic.WORKLOADS[1]
    W, M, G, V = bench.build_inputs(wl, torch, np, synthetic, torch.device("cpu"))
    assert len(W) == len(M) == len(G) == len(V) == wl.n_matrices
    for (idx, r, c), w, m, g, v in zip(wl.matrices(), W, M, G, V):
        assert w.shape == m.shape == g.shape == (r, c) and v.shape == (r,)
        assert m.dtype == torch.float32 and not torch.any(m) and not torch.any(w)
        ref = synthetic.gradient(wl.dist, r, c, wl.storage, wl.index, 0, idx)
        assert np.array_equal(g.numpy(), ref)


def test_build_inputs_bf16_bits_preserved():
    # a bf16 workload cut to two small matrices: the device copies keep the gradient's bits
    wl = dataclasses.replace(synthetic.WORKLOADS[2], groups=(synthetic.configs.MatrixSpec(64, 192, 2),))
    W, M, G, V = bench.build_inputs(wl, torch, np, synthetic, torch.device("cpu"))
    for (idx, r, c), w, g in zip(wl.matrices(), W, G):
        assert g.dtype == torch.bfloat16 and w.dtype == torch.bfloat16
        ref = synthetic.gradient(wl.dist, r, c, "bf16", wl.index, 0, idx)
        assert np.array_equal(g.view(torch.int16).numpy().view(np.uint16), ref.view(np.uint16))


def test_traffic_lookup_unknown_kernel_is_none():
    assert bench.measured_traffic("no_such_kernel", "config2-standard") is None


def test_dense_equivalent_counts():
    # T (4 m n^2 + 2 n^3) per matrix, summed: 4 x 4096^2 -> 8.25e12, 4096x16384 -> 6.18e12,
    # the 196-matrix layer set -> 2.516e14 (tall matrices counted on their short side)
    assert abs(bench.dense_equivalent_flops(synthetic.WORKLOADS[2]) / 8.246e12 - 1) < 1e-3
    assert abs(bench.dense_equivalent_flops(synthetic.WORKLOADS[3]) / 6.185e12 - 1) < 1e-3
    assert abs(bench.dense_equivalent_flops(synthetic.WORKLOADS[4]) / 2.516e14 - 1) < 1e-3
    # Dion3 orthogonalises k = ceil(f rows) rows
    assert bench.ns_shapes(synthetic.WORKLOADS[5]) == [(1280, 13824)]


def test_default_workload_is_the_layer_set():
    args = bench.parse([])
    assert args.workload == 4 and synthetic.WORKLOADS[4].n_matrices == 196
    assert bench.parse(["--config", "2"]).workload == 2


def test_parallel_gradients_equal_serial():
    wl = dataclasses.replace(synthetic.WORKLOADS[4], groups=(synthetic.configs.MatrixSpec(64, 96, 3),
                                                             synthetic.configs.MatrixSpec(96, 64, 2)))
    got = list(bench.gradient_bits(wl, synthetic, threads=4))
    for (idx, r, c), g in zip(wl.matrices(), got):
        assert np.array_equal(g, synthetic.gradient(wl.dist, r, c, wl.storage, wl.index, 0, idx))


def test_host_info_fields():
    info, threads = bench.host_info()
    assert info["os_cpu_count"] == os.cpu_count()
    assert "cpu_model" in info and "blas" in info


def test_clock_sampler_reports_fields_without_a_device():
    c = bench.ClockSampler()
    c.sample()
    s = c.summary()
    assert set(s) == {"sys_clock_mhz", "mem_clock_mhz", "socket_power_w", "samples", "window_s",
                      "reliable", "source"}
