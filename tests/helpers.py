"""Test-side helpers: moving stored bits between NumPy and torch, and the comparison rules.

Tolerances (relative Frobenius error per matrix, after each step): 1e-4 when W, G, X are
float32 and 2e-2 when they are bfloat16.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_device(stored: np.ndarray, storage: str, device="cuda") -> torch.Tensor:
    if storage == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact float64 values (bfloat16 widened by the oracle's decoder)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def stored_f64(stored: np.ndarray, storage: str) -> np.ndarray:
    if storage == "bf16":
        return oracle.bf16_bits_to_f64(stored)
    return np.asarray(stored, dtype=np.float64)


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def ulp_half(w: np.ndarray, storage: str) -> np.ndarray:
    """Half the spacing of the storage format at |w| (the bound of one rounding)."""
    w = np.abs(np.asarray(w, dtype=np.float64))
    mant_bits = 8 if storage == "bf16" else 24
    e = np.floor(np.log2(np.maximum(w, 2.0 ** -126)))
    return 0.5 * 2.0 ** (e - (mant_bits - 1))


def check_weight(W_gpu, W0, delta_ref, storage: str, what: str = "W") -> float:
    """W_gpu = round(W0 + delta_gpu) with ||delta_gpu - delta_ref|| <= tol ||delta_ref||, so
    ||W_gpu - W0 - delta_ref|| <= tol ||delta_ref|| + ||ulp/2|| (one rounding per element)."""
    W_gpu = np.asarray(W_gpu, dtype=np.float64)
    err = np.linalg.norm(W_gpu - W0 - delta_ref)
    bound = TOL[storage] * np.linalg.norm(delta_ref) + np.linalg.norm(ulp_half(W0 + delta_ref, storage))
    assert err <= bound, f"{what}: |W - W0 - delta| = {err:.4g} > bound {bound:.4g}"
    return float(err / max(np.linalg.norm(delta_ref), 1e-300))


def dion3_rows_used(M0, G, M1, W0, W1, k: int, what: str = "") -> np.ndarray:
    """The rows a Dion3 step on the GPU selected, for re-running the oracle on them.

    A selected row is decayed (M1 differs from float32(M0 + G), the one rounding an
    unselected row gets) or updated (W1 differs from W0). The GPU ranks float32 l1 norms,
    the oracle float64 ones: a row may differ from the oracle's choice only where its
    float64 norm lies within 1e-5 relative of the k-th largest."""
    Mg = np.asarray(M0, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    Mg32 = Mg.astype(np.float32).astype(np.float64)
    sel_gpu = np.where(np.any(np.asarray(M1) != Mg32, axis=1) |
                       np.any(np.asarray(W1) != np.asarray(W0), axis=1))[0]
    S_orc = oracle.select_rows(Mg, k)
    l1 = np.abs(Mg).sum(axis=1)
    kth = np.sort(l1)[::-1][k - 1]
    diff = np.setxor1d(sel_gpu, S_orc)
    assert all(abs(l1[i] - kth) <= 1e-5 * kth for i in diff), (what, diff[:10])
    rows = sel_gpu if len(diff) else S_orc
    assert len(rows) == k, (what, len(rows), k)
    return np.sort(rows)
