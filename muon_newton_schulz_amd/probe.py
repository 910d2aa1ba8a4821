"""ctypes binding of libmns_probe.so (include/mns_probe.h): the MFMA-only ceiling probe.

A measurement aid for bench.py, not part of the optimizer path: one kernel of back-to-back
v_mfma_f32_32x32x16_f16 on every compute unit, no memory traffic in its loop, so its rate is
the most the matrix pipes deliver at the clock the part holds under that load.
"""
from __future__ import annotations

import ctypes
import os

PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmns_probe.so")

# Every symbol include/mns_probe.h declares.
EXPORTS = ("mns_probe_mfma_launch", "mns_probe_mfma_checksum")

_lib = None


def load(path: str | None = None):
    """Load the probe library (built in-tree by muon_newton_schulz_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or PROBE_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with python -m muon_newton_schulz_amd.build")
    lib = ctypes.CDLL(p)
    lib.mns_probe_mfma_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_double)]
    lib.mns_probe_mfma_launch.restype = ctypes.c_int
    lib.mns_probe_mfma_checksum.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.mns_probe_mfma_checksum.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def mfma_launch(iters: int, zero_operands: bool = False, stream=None) -> float:
    """Enqueue one probe launch on `stream` (a torch stream, or None for the null stream);
    returns its float16 FLOPs."""
    lib = load()
    flops = ctypes.c_double(0.0)
    handle = ctypes.c_void_p(stream.cuda_stream if stream is not None else 0)
    rc = lib.mns_probe_mfma_launch(int(iters), 1 if zero_operands else 0, handle,
                                   ctypes.byref(flops))
    if rc != 0:
        raise RuntimeError(f"mns_probe_mfma_launch failed with status {rc}")
    return flops.value


def mfma_checksum(n: int = 4096) -> float:
    """Sum of the absolute values of the first `n` per-thread results of the last launch
    (synchronises the device)."""
    lib = load()
    s = ctypes.c_double(0.0)
    rc = lib.mns_probe_mfma_checksum(int(n), ctypes.byref(s))
    if rc != 0:
        raise RuntimeError(f"mns_probe_mfma_checksum failed with status {rc}")
    return s.value
