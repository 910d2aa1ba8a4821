"""MI355X (gfx950) Muon / Newton-Schulz / Gram-NS / NorMuon / Dion3 optimizer step.

Thin Python binding over the C ABI in include/muon_ns.h: it turns torch tensors into
device pointers and sizes and calls the HIP library; every step of the computation runs in
the library's kernels. PyTorch supplies device memory and the current stream only. The
library must be built (``python -m muon_newton_schulz_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import Iterable, Sequence

import torch

from . import _abi
from ._abi import (MNS_BF16, MNS_F32, MNS_NS_GRAM, MNS_NS_STANDARD, MnsError,  # noqa: F401
                   MnsHparams, MnsMatrix, check, load)

__all__ = ["muon_step", "ns_orthogonalize", "gram_ns_orthogonalize", "normuon_scale",
           "step_workspace_size", "ns_workspace_size", "normuon_workspace_size",
           "restart_mask", "profile_begin", "profile_end", "MnsError", "load"]

_KINDS = {"standard": MNS_NS_STANDARD, "gram": MNS_NS_GRAM}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MNS_BF16
    if t.dtype == torch.float32:
        return MNS_F32
    raise TypeError(f"unsupported storage dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _coeffs(coeffs: Sequence[Sequence[float]]):
    flat = [float(c) for abc in coeffs for c in abc]
    if len(flat) != 3 * len(coeffs):
        raise ValueError("each iteration needs (a_t, b_t, c_t)")
    return (ctypes.c_float * max(1, len(flat)))(*flat), len(coeffs)


def restart_mask(restart_before: Iterable[int]) -> int:
    """Bit t set = restart before iteration t (Gram Newton-Schulz)."""
    mask = 0
    for t in restart_before:
        mask |= 1 << int(t)
    return mask


def _workspace(nbytes: int, device, workspace: torch.Tensor | None) -> torch.Tensor:
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _as_list(x):
    if x is None:
        return None
    return list(x) if isinstance(x, (list, tuple)) else [x]


def _hparams(dtype: int, mu, lr, coeffs, kind, restart_before, normuon, beta2, eps,
             row_fraction):
    abc, T = _coeffs(coeffs)
    hp = MnsHparams(mu=mu, lr=lr, T=T, abc=ctypes.cast(abc, ctypes.POINTER(ctypes.c_float)),
                    kind=_KINDS[kind], restart_mask=restart_mask(restart_before),
                    normuon=1 if normuon else 0, beta2=beta2, eps=eps,
                    row_fraction=row_fraction, dtype=dtype)
    return hp, abc


def _matrices(W, M, G, v):
    Ws, Ms, Gs, vs = _as_list(W), _as_list(M), _as_list(G), _as_list(v)
    if not (len(Ws) == len(Ms) == len(Gs)) or (vs is not None and len(vs) != len(Ws)):
        raise ValueError("W, M, G (and v) must have the same number of matrices")
    arr = (MnsMatrix * len(Ws))()
    for i, (w, m, g) in enumerate(zip(Ws, Ms, Gs)):
        if w.dim() != 2 or w.shape != m.shape or w.shape != g.shape:
            raise ValueError("W, M and G must be 2-D tensors of the same shape")
        if m.dtype != torch.float32:
            raise TypeError("momentum must be float32")
        arr[i].W = _ptr(w)
        arr[i].M = _ptr(m)
        arr[i].G = _ptr(g)
        arr[i].v = _ptr(vs[i]) if vs is not None else None
        arr[i].rows, arr[i].cols = w.shape
    return arr, Ws


def step_workspace_size(W, M, G, v=None, *, mu=0.95, lr=0.02, coeffs, kind="standard",
                        restart_before=(), normuon=False, beta2=0.95, eps=1e-8,
                        row_fraction=1.0) -> int:
    arr, Ws = _matrices(W, M, G, v)
    hp, _keep = _hparams(_dtype_code(Ws[0]), mu, lr, coeffs, kind, restart_before, normuon,
                         beta2, eps, row_fraction)
    out = ctypes.c_size_t(0)
    check(load().mns_step_workspace_size(arr, len(Ws), ctypes.byref(hp), ctypes.byref(out)),
          "mns_step_workspace_size")
    return out.value


def muon_step(W, M, G, v=None, *, mu: float, lr: float, coeffs, kind: str = "standard",
              restart_before=(), normuon: bool = False, beta2: float = 0.95,
              eps: float = 1e-8, row_fraction: float = 1.0,
              workspace: torch.Tensor | None = None, stream=None) -> None:
    """One optimizer step, in place on W, M (and v), over one matrix or a list of them.

    Eq. (1) of the Dion3 page; NorMuon (Eq. 2) when ``normuon``; Dion3 fractional row
    selection (Algorithm 4) when ``row_fraction`` < 1 (``lr`` is used as given)."""
    lib = load()
    arr, Ws = _matrices(W, M, G, v)
    hp, _keep = _hparams(_dtype_code(Ws[0]), mu, lr, coeffs, kind, restart_before, normuon,
                         beta2, eps, row_fraction)
    need = ctypes.c_size_t(0)
    check(lib.mns_step_workspace_size(arr, len(Ws), ctypes.byref(hp), ctypes.byref(need)),
          "mns_step_workspace_size")
    ws = _workspace(need.value, Ws[0].device, workspace)
    check(lib.muon_step(arr, len(Ws), ctypes.byref(hp), ws.data_ptr(),
                        ws.numel() * ws.element_size(), _stream(stream)), "muon_step")


def ns_workspace_size(X: torch.Tensor, kind: str = "standard") -> int:
    b, r, c = _bshape(X)
    out = ctypes.c_size_t(0)
    check(load().mns_ns_workspace_size(_dtype_code(X), b, r, c, _KINDS[kind],
                                       ctypes.byref(out)), "mns_ns_workspace_size")
    return out.value


def _bshape(X: torch.Tensor):
    if X.dim() == 2:
        return 1, X.shape[0], X.shape[1]
    if X.dim() == 3:
        return X.shape[0], X.shape[1], X.shape[2]
    raise ValueError("X must be 2-D or a 3-D batch")


def ns_orthogonalize(X: torch.Tensor, coeffs, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Standard quintic Newton-Schulz of X / ||X||_F (per matrix of a batch)."""
    lib = load()
    b, r, c = _bshape(X)
    O = torch.empty_like(X) if out is None else out
    abc, T = _coeffs(coeffs)
    ws = _workspace(ns_workspace_size(X, "standard"), X.device, workspace)
    check(lib.ns_orthogonalize(_ptr(X), _ptr(O), _dtype_code(X), b, r, c, T, abc,
                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
          "ns_orthogonalize")
    return O


def gram_ns_orthogonalize(X: torch.Tensor, coeffs, restart_before=(3,),
                          out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Gram Newton-Schulz (Theorem 2 with restarts) of X / ||X||_F."""
    lib = load()
    b, r, c = _bshape(X)
    O = torch.empty_like(X) if out is None else out
    abc, T = _coeffs(coeffs)
    ws = _workspace(ns_workspace_size(X, "gram"), X.device, workspace)
    check(lib.gram_ns_orthogonalize(_ptr(X), _ptr(O), _dtype_code(X), b, r, c, T, abc,
                                    restart_mask(restart_before), ws.data_ptr(),
                                    ws.numel() * ws.element_size(), _stream(stream)),
          "gram_ns_orthogonalize")
    return O


def normuon_workspace_size(O: torch.Tensor) -> int:
    b, r, c = _bshape(O)
    out = ctypes.c_size_t(0)
    check(load().mns_normuon_workspace_size(b, r, c, ctypes.byref(out)),
          "mns_normuon_workspace_size")
    return out.value


def normuon_scale(O: torch.Tensor, v: torch.Tensor, beta2: float = 0.95, eps: float = 1e-8,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """NorMuon normalisation (Eq. 2) of O in place; v (float32, one per row) is updated."""
    lib = load()
    b, r, c = _bshape(O)
    if v.dtype != torch.float32 or v.numel() != b * r:
        raise ValueError("v must be float32 with one entry per row")
    ws = _workspace(normuon_workspace_size(O), O.device, workspace)
    check(lib.normuon_scale(_ptr(O), _dtype_code(O), b, r, c,
                            ctypes.cast(_ptr(v), ctypes.POINTER(ctypes.c_float)), beta2, eps,
                            ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
          "normuon_scale")
    return O


def profile_begin() -> None:
    """Start bracketing every library kernel launch with hipEvents (see mns_profile_begin)."""
    check(load().mns_profile_begin(), "mns_profile_begin")


def profile_end() -> list[dict]:
    """Close the session; per kernel: launches, event ms, algorithmic FLOPs and bytes."""
    lib = load()
    cap = 64
    arr = (_abi.MnsKernelStat * cap)()
    n = ctypes.c_int(0)
    check(lib.mns_profile_end(arr, cap, ctypes.byref(n)), "mns_profile_end")
    return [{"name": arr[i].name.decode(), "launches": arr[i].launches, "ms": arr[i].ms,
             "flops": arr[i].flops, "bytes": arr[i].bytes} for i in range(min(n.value, cap))]
