"""Build the HIP libraries (gfx950) in-tree: muon_newton_schulz_amd/libmuon_ns.so (the
optimizer step) and muon_newton_schulz_amd/libmns_probe.so (the MFMA ceiling probe, a
measurement aid).

Usage: python -m muon_newton_schulz_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmuon_ns.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["abi.cpp", "elementwise.hip", "gemm.hip"]
PROBE_NAME = "libmns_probe.so"
PROBE_PATH = os.path.join(PKG, PROBE_NAME)
PROBE_SOURCES = ["probe.hip"]

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep hipcc from forming packed-FP32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile_link(cc, sources, out_path, verbose, extra_flags):
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in sources:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
               "-x", "hip", "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
        noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if verbose and noise:
            print("\n".join(noise))
        objs.append(obj)
    tmp = out_path + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out_path)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source for gfx950 and link both shared libraries. Returns the path of
    the optimizer-step library."""
    cc = hipcc()
    _compile_link(cc, SOURCES, LIB_PATH, verbose, extra_flags)
    _compile_link(cc, PROBE_SOURCES, PROBE_PATH, verbose, extra_flags)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
