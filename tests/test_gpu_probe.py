"""The MFMA-only ceiling probe (libmns_probe.so, a measurement aid of bench.py) on a GPU: it
runs, zero operands give zero results, the results grow linearly with the iteration count
(the loop really accumulates), and its rate stays within the hardware's published peak."""
import math

import pytest

pytestmark = pytest.mark.gpu


def test_probe_accumulates_and_rate_is_physical():
    import torch
    from muon_newton_schulz_amd import probe

    print("probe: zero operands, 200 iterations", flush=True)
    probe.mfma_launch(200, zero_operands=True)
    assert probe.mfma_checksum(4096) == 0.0

    print("probe: random operands, 100 and 200 iterations", flush=True)
    probe.mfma_launch(100)
    s1 = probe.mfma_checksum(4096)
    probe.mfma_launch(200)
    s2 = probe.mfma_checksum(4096)
    assert math.isfinite(s1) and s1 > 0.0
    # every accumulator is iters x (the same sum of products): twice the iterations, twice
    # the absolute values (float32 accumulation over 200 steps: rounding well below 1e-3)
    assert abs(s2 / s1 - 2.0) < 1e-3, (s1, s2)

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe.mfma_launch(2000, stream=stream)   # warm
    e0.record(stream)
    flops = probe.mfma_launch(2000, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"probe: {tflops:.1f} TFLOP/s", flush=True)
    assert 100.0 < tflops <= 1.05 * 2500.0
