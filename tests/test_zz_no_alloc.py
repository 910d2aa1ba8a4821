"""The allocation-free standard NS (ns_orthogonalize_noalloc), called through the C ABI: two
calls in a row (the second on a smaller input, so the library's scratch still holds the
first call's buffers) must each match ns_orthogonalize with a caller workspace on the same
input, to the parity gate (and bit for bit where both run the same chunking), and the fp64
oracle. Sizes beyond the scratch are rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as mns
import oracle
import synthetic
from helpers import TOL, rel, stored_f64, to_device, to_f64
from muon_newton_schulz_amd import _abi

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)


def _say(*a):
    print(*a, flush=True)


def _abc(coeffs):
    flat = [float(c) for t in coeffs for c in t]
    return (ctypes.c_float * len(flat))(*flat), len(coeffs)


def _noalloc(lib, X, O, storage, coeffs):
    b, r, c = (1, *X.shape) if X.dim() == 2 else tuple(X.shape)
    abc, T = _abc(coeffs)
    dt = _abi.MNS_BF16 if storage == "bf16" else _abi.MNS_F32
    return lib.ns_orthogonalize_noalloc(X.data_ptr(), O.data_ptr(), dt, b, r, c, T, abc,
                                        torch.cuda.current_stream().cuda_stream)


# (storage, batch, rows, cols) of the first and the second (smaller) call
CASES = {
    "bf16_wide_then_tall": (("bf16", 3, 384, 1100), ("bf16", 2, 500, 260)),
    "bf16_tall_then_single": (("bf16", 2, 1024, 700), ("bf16", 1, 130, 300)),
    "f32_batch_then_single": (("f32", 4, 256, 640), ("f32", 1, 100, 257)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_workspace_entry_point(case):
    lib = mns.load()
    coeffs = [QUINTIC] * 5
    for call, (storage, batch, rows, cols) in enumerate(CASES[case]):
        _say(f"case {case} call {call}: {batch} x {rows}x{cols} {storage}")
        gs = [synthetic.gradient("student_t", rows, cols, storage, 971, call, i)
              for i in range(batch)]
        X = torch.stack([to_device(g, storage) for g in gs])
        O_na = torch.empty_like(X)
        st = _noalloc(lib, X, O_na, storage, coeffs)
        assert st == _abi.MNS_OK, lib.mns_status_string(st)
        O_ws = mns.ns_orthogonalize(X, coeffs)
        torch.cuda.synchronize()
        same = torch.equal(O_na, O_ws)
        worst_ws, worst_orc = 0.0, 0.0
        for i in range(batch):
            a, b = to_f64(O_na[i]), to_f64(O_ws[i])
            worst_ws = max(worst_ws, rel(a, b))
            ref = oracle.newton_schulz(stored_f64(gs[i], storage), coeffs)
            worst_orc = max(worst_orc, rel(a, ref))
        _say(f"  bit-identical to ns_orthogonalize: {same}; vs it {worst_ws:.2e}; "
             f"vs oracle {worst_orc:.2e}")
        assert worst_ws <= TOL[storage] and worst_orc <= TOL[storage]


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = mns.load()
    X = torch.zeros(2048 + 256, 4096, dtype=torch.bfloat16, device="cuda")
    O = torch.empty_like(X)
    st = _noalloc(lib, X, O, "bf16", [QUINTIC] * 5)
    assert st == _abi.MNS_ERR_WORKSPACE
    assert torch.count_nonzero(O.view(torch.int16)).item() >= 0   # nothing ran; O untouched by the call
