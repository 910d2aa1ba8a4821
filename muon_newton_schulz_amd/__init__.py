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

__all__ = ["muon_step", "ns_orthogonalize", "ns_orthogonalize_noalloc",
           "gram_ns_orthogonalize", "normuon_scale",
           "step_workspace_size", "ns_workspace_size", "normuon_workspace_size",
           "restart_mask", "profile_begin", "profile_set_flush", "profile_end", "MnsError",
           "load"]

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


def _on_one_gpu(tensors, what: str) -> torch.device:
    """Every tensor must live on one CUDA (HIP) device: a host pointer handed to a kernel
    faults the GPU. Returns that device."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{what}: every tensor must be on a GPU (got {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{what}: tensors on different devices ({dev} and {t.device})")
    return dev


def _span(t: torch.Tensor):
    n = t.numel() * t.element_size()
    return t.data_ptr(), t.data_ptr() + n


def _disjoint(a: torch.Tensor, b: torch.Tensor) -> bool:
    a0, a1 = _span(a)
    b0, b1 = _span(b)
    return a1 <= b0 or b1 <= a0


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _coeffs(coeffs: Sequence[Sequence[float]]):
    flat = [float(c) for abc in coeffs for c in abc]
    if len(flat) != 3 * len(coeffs):
        raise ValueError("each iteration needs (a_t, b_t, c_t)")
    return (ctypes.c_float * max(1, len(flat)))(*flat), len(coeffs)


# The restart mask is a 32-bit field: restarts can be placed before iterations 2 .. 31.
MAX_RESTART_ITERATION = 31


def restart_mask(restart_before: Iterable[int], T: int | None = None) -> int:
    """Bit t set = restart before iteration t (Gram Newton-Schulz). Raises for an iteration
    outside 2 .. min(T, 31) (T given) or 2 .. 31."""
    hi = MAX_RESTART_ITERATION if T is None else min(int(T), MAX_RESTART_ITERATION)
    mask = 0
    for t in restart_before:
        t = int(t)
        if not 2 <= t <= hi:
            raise ValueError(f"restart before iteration {t}: must lie in 2..{hi}")
        mask |= 1 << t
    return mask


def _workspace(nbytes: int, device, workspace: torch.Tensor | None) -> torch.Tensor:
    if workspace is not None:
        if workspace.device != device:
            raise ValueError(f"workspace on {workspace.device}, tensors on {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
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
    if kind not in _KINDS:
        raise ValueError(f"kind must be one of {sorted(_KINDS)}")
    hp = MnsHparams(mu=mu, lr=lr, T=T, abc=ctypes.cast(abc, ctypes.POINTER(ctypes.c_float)),
                    kind=_KINDS[kind], restart_mask=restart_mask(restart_before, T),
                    normuon=1 if normuon else 0, beta2=beta2, eps=eps,
                    row_fraction=row_fraction, dtype=dtype)
    return hp, abc


def _first_dtype(W) -> int:
    Ws = _as_list(W)
    if not Ws:
        raise ValueError("no matrices")
    return _dtype_code(Ws[0])


def _matrices(W, M, G, v, normuon: bool):
    """Checks the step's tensors and packs them into the ABI's matrix array. The library
    applies one storage dtype to every W and G of a call and reads v as float32 [rows], so
    a mismatch here would make its kernels read or write out of bounds."""
    Ws, Ms, Gs, vs = _as_list(W), _as_list(M), _as_list(G), _as_list(v)
    if not Ws:
        raise ValueError("no matrices")
    if not (len(Ws) == len(Ms) == len(Gs)) or (vs is not None and len(vs) != len(Ws)):
        raise ValueError("W, M, G (and v) must have the same number of matrices")
    if normuon and vs is None:
        raise ValueError("NorMuon needs v (one float32 vector per matrix)")
    dtype = Ws[0].dtype
    _dtype_code(Ws[0])
    for i, (w, m, g) in enumerate(zip(Ws, Ms, Gs)):
        if w.dim() != 2 or w.shape != m.shape or w.shape != g.shape:
            raise ValueError(f"matrix {i}: W, M and G must be 2-D tensors of the same shape")
        if w.dtype != dtype or g.dtype != dtype:
            raise TypeError(f"matrix {i}: W and G must all share one storage dtype ({dtype}); "
                            f"got W {w.dtype}, G {g.dtype}")
        if m.dtype != torch.float32:
            raise TypeError(f"matrix {i}: momentum must be float32")
        if vs is not None:
            vi = vs[i]
            if vi.dtype != torch.float32 or vi.dim() != 1 or vi.shape[0] != w.shape[0]:
                raise ValueError(f"matrix {i}: v must be float32 of shape ({w.shape[0]},)")
        for t in (w, m, g) + ((vs[i],) if vs is not None else ()):
            if not t.is_contiguous():
                raise ValueError(f"matrix {i}: tensors must be contiguous")
    dev = _on_one_gpu(Ws + Ms + Gs + (vs or []), "muon_step")
    arr = (MnsMatrix * len(Ws))()
    for i, (w, m, g) in enumerate(zip(Ws, Ms, Gs)):
        arr[i].W = _ptr(w)
        arr[i].M = _ptr(m)
        arr[i].G = _ptr(g)
        arr[i].v = _ptr(vs[i]) if vs is not None else None
        arr[i].rows, arr[i].cols = w.shape
    return arr, Ws, dev


def step_workspace_size(W, M, G, v=None, *, mu=0.95, lr=0.02, coeffs, kind="standard",
                        restart_before=(), normuon=False, beta2=0.95, eps=1e-8,
                        row_fraction=1.0) -> int:
    hp, _keep = _hparams(_first_dtype(W), mu, lr, coeffs, kind, restart_before, normuon,
                         beta2, eps, row_fraction)
    arr, Ws, _dev = _matrices(W, M, G, v, normuon)
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
    hp, _keep = _hparams(_first_dtype(W), mu, lr, coeffs, kind, restart_before, normuon,
                         beta2, eps, row_fraction)
    arr, Ws, dev = _matrices(W, M, G, v, normuon)
    lib = load()
    need = ctypes.c_size_t(0)
    check(lib.mns_step_workspace_size(arr, len(Ws), ctypes.byref(hp), ctypes.byref(need)),
          "mns_step_workspace_size")
    ws = _workspace(need.value, dev, workspace)
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


def _ns_operands(X: torch.Tensor, out: torch.Tensor | None, what: str):
    """X (2-D, or a 3-D batch) in a storage dtype on one GPU, and the output: a new tensor
    like X, or `out`, which must match X in shape, dtype and device and not overlap it."""
    b, r, c = _bshape(X)
    _dtype_code(X)
    if not X.is_contiguous():
        raise ValueError(f"{what}: X must be contiguous")
    if out is not None:
        if out.shape != X.shape or out.dtype != X.dtype:
            raise ValueError(f"{what}: out must match X in shape and dtype "
                             f"(X {tuple(X.shape)} {X.dtype}, out {tuple(out.shape)} {out.dtype})")
        if not out.is_contiguous():
            raise ValueError(f"{what}: out must be contiguous")
    if out is not None and not _disjoint(X, out):
        raise ValueError(f"{what}: out may not overlap X")
    _on_one_gpu([X, out], what)
    O = torch.empty_like(X) if out is None else out
    return b, r, c, O


def ns_orthogonalize(X: torch.Tensor, coeffs, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Standard quintic Newton-Schulz of X / ||X||_F (per matrix of a batch)."""
    b, r, c, O = _ns_operands(X, out, "ns_orthogonalize")
    abc, T = _coeffs(coeffs)
    lib = load()
    ws = _workspace(ns_workspace_size(X, "standard"), X.device, workspace)
    check(lib.ns_orthogonalize(_ptr(X), _ptr(O), _dtype_code(X), b, r, c, T, abc,
                               ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
          "ns_orthogonalize")
    return O


def ns_orthogonalize_noalloc(X: torch.Tensor, coeffs, out: torch.Tensor, stream=None) -> torch.Tensor:
    """ns_orthogonalize without a workspace: the library's own device scratch (64 MiB per GPU)
    holds every buffer, so the call allocates nothing (graph capture, serving loops). `out`
    must be given; overlapping calls on one GPU race."""
    if out is None:
        raise ValueError("ns_orthogonalize_noalloc: out must be given (nothing is allocated)")
    b, r, c, O = _ns_operands(X, out, "ns_orthogonalize_noalloc")
    abc, T = _coeffs(coeffs)
    check(load().ns_orthogonalize_noalloc(_ptr(X), _ptr(O), _dtype_code(X), b, r, c, T, abc,
                                          _stream(stream)), "ns_orthogonalize_noalloc")
    return O


def gram_ns_orthogonalize(X: torch.Tensor, coeffs, restart_before=(3,),
                          out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Gram Newton-Schulz (Theorem 2 with restarts) of X / ||X||_F."""
    b, r, c, O = _ns_operands(X, out, "gram_ns_orthogonalize")
    abc, T = _coeffs(coeffs)
    mask = restart_mask(restart_before, T)
    lib = load()
    ws = _workspace(ns_workspace_size(X, "gram"), X.device, workspace)
    check(lib.gram_ns_orthogonalize(_ptr(X), _ptr(O), _dtype_code(X), b, r, c, T, abc,
                                    mask, ws.data_ptr(),
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
    b, r, c = _bshape(O)
    _dtype_code(O)
    if v.dtype != torch.float32 or v.numel() != b * r:
        raise ValueError("v must be float32 with one entry per row")
    if not O.is_contiguous() or not v.is_contiguous():
        raise ValueError("normuon_scale: O and v must be contiguous")
    if not _disjoint(O, v):
        raise ValueError("normuon_scale: v may not overlap O")
    _on_one_gpu([O, v], "normuon_scale")
    lib = load()
    ws = _workspace(normuon_workspace_size(O), O.device, workspace)
    check(lib.normuon_scale(_ptr(O), _dtype_code(O), b, r, c,
                            ctypes.cast(_ptr(v), ctypes.POINTER(ctypes.c_float)), beta2, eps,
                            ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
          "normuon_scale")
    return O


def profile_begin() -> None:
    """Start bracketing every library kernel launch with hipEvents (see mns_profile_begin)."""
    check(load().mns_profile_begin(), "mns_profile_begin")


def profile_set_flush(buffer: torch.Tensor | None) -> None:
    """Flush caches before each HBM-bound launch of the open session by writing over
    `buffer` (a device tensor, >= 1 GiB to evict the Infinity Cache); None turns it off."""
    if buffer is None:
        check(load().mns_profile_set_flush(None, 0), "mns_profile_set_flush")
        return
    if buffer.device.type != "cuda" or not buffer.is_contiguous():
        raise ValueError("the flush buffer must be a contiguous GPU tensor")
    check(load().mns_profile_set_flush(buffer.data_ptr(), buffer.numel() * buffer.element_size()),
          "mns_profile_set_flush")


def profile_end() -> list[dict]:
    """Close the session; per kernel: launches, event ms, algorithmic FLOPs and bytes."""
    lib = load()
    cap = 64
    arr = (_abi.MnsKernelStat * cap)()
    n = ctypes.c_int(0)
    check(lib.mns_profile_end(arr, cap, ctypes.byref(n)), "mns_profile_end")
    return [{"name": arr[i].name.decode(), "launches": arr[i].launches, "ms": arr[i].ms,
             "flops": arr[i].flops, "bytes": arr[i].bytes} for i in range(min(n.value, cap))]
