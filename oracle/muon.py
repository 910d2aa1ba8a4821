"""fp64 reference implementation of the Muon-family optimizer step.

TEST INFRASTRUCTURE ONLY -- see the package docstring. Source of every formula: the page
"Dion3: Full-stack orthogonal updates" (arXiv 2608.11612). Section names below are that
page's.

Conventions (readings where the page is silent; each is listed with its reason in the
repository's design notes):
* A matrix is handled as ``n x m`` with ``n <= m`` (aspect ratio ``alpha = m/n >= 1``,
  section "Standard Newton-Schulz", FLOP analysis). A stored tall matrix is processed
  through its transpose, which is exact because ``polar(X^T) = polar(X)^T``.
* ``||X||_F = 0`` gives a zero orthogonalised output (the polar factor of the zero matrix
  is taken as zero) and the NorMuon ratio ``0/0`` is taken as 0.
* NorMuon: ``v`` starts at 0, no bias correction, epsilon added after the square root,
  "row" is a stored row of ``W`` and ``m`` its length.
* Gram Newton-Schulz restart "at t = 3" means: before iteration 3, form ``X_2 = Q_2 X``,
  recompute the Gram matrix from it and reset ``Q`` to the identity.
* Dion3: the gradient enters as ``M <- M + G`` before selection; afterwards only the
  selected rows are decayed by ``mu``; top-k ties go to the lower row index.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "FlopCounter", "bf16_bits_to_f64", "f64_to_bf16_bits", "round_to_storage", "frobenius",
    "polar_svd", "newton_schulz", "gram_newton_schulz", "orthogonalize", "normuon_update", "muon_step",
    "select_rows", "dion3_step", "rows_for_fraction", "transfer_lr",
    "flops_standard_formula", "flops_standard_symmetric_formula", "flops_gram_formula",
    "flops_restart_formula",
]


# --------------------------------------------------------------------------------------
# Storage encodings (not part of the method: how the stored inputs/outputs are read)
# --------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) exactly to float64.

    A bfloat16 value is the upper half of an IEEE binary32 word, so shifting the 16 bits
    into the top of a 32-bit word and reading it as binary32 is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


_BF16_MAX = float.fromhex("0x1.fep127")      # largest finite bfloat16
_BF16_MIN_NORMAL = 2.0 ** -126


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16, round-to-nearest-even, returning uint16 bits.

    Written directly from the binary format (8 exponent bits, 7 stored fraction bits):
    a normal value keeps 8 significant bits; below the smallest normal the spacing is
    2^-133. Rounding is a single step from the exact float64 value."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    sign = np.signbit(flat)
    ax = np.abs(flat)
    nan = np.isnan(flat)
    with np.errstate(invalid="ignore", over="ignore"):
        mant, expo = np.frexp(ax)                  # ax = mant * 2**expo, mant in [0.5, 1)
        normal = ax >= _BF16_MIN_NORMAL
        q_norm = np.rint(mant * 256.0)             # 8 significant bits, half to even
        v_norm = np.ldexp(q_norm, expo - 8)
        v_sub = np.rint(ax * 2.0 ** 133) * 2.0 ** -133
        val = np.where(normal, v_norm, v_sub)
        val = np.where(np.isinf(ax) | (val > _BF16_MAX), np.inf, val)
        f32 = val.astype(np.float32)               # exact: val has <= 8 significant bits
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(sign, bits | np.uint16(0x8000), bits)
    bits = np.where(nan, np.uint16(0x7FC0), bits)
    out[:] = bits
    return out.reshape(x.shape)


def round_to_storage(x, storage: str) -> np.ndarray:
    """Round float64 values to the storage type ('f32' or 'bf16') and widen back."""
    x = np.asarray(x, dtype=np.float64)
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)   # IEEE round-to-nearest-even
    if storage == "bf16":
        return bf16_bits_to_f64(f64_to_bf16_bits(x))
    raise ValueError(f"unknown storage type {storage!r}")


def frobenius(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.sum(x * x)))


# --------------------------------------------------------------------------------------
# FLOP accounting (section "Standard Newton-Schulz", FLOP analysis; section
# "1. Gram Newton-Schulz", FLOP analysis and restart cost)
# --------------------------------------------------------------------------------------

class FlopCounter:
    """Counts the matrix products the oracle executes.

    ``dense`` counts 2*M*N*K per product. ``algorithmic`` counts a product whose result
    is symmetric at half that (the page prices a symmetric GEMM at n^3 for an n x n x n
    product), which is the work a symmetric kernel must do."""

    def __init__(self):
        self.dense = 0
        self.algorithmic = 0
        self.products: list[tuple[int, int, int, bool]] = []

    def record(self, m: int, n: int, k: int, symmetric: bool) -> None:
        self.dense += 2 * m * n * k
        self.algorithmic += (m * n * k) if symmetric else (2 * m * n * k)
        self.products.append((m, n, k, symmetric))


def _mm(p: np.ndarray, q: np.ndarray, counter: FlopCounter | None, symmetric: bool = False):
    if counter is not None:
        counter.record(p.shape[0], q.shape[1], p.shape[1], symmetric)
    return p @ q


def flops_standard_formula(n: int, m: int, T: int) -> int:
    """Dense standard-NS cost T(4mn^2 + 2n^3) (section "Standard Newton-Schulz")."""
    return T * (4 * m * n * n + 2 * n ** 3)


def flops_standard_symmetric_formula(n: int, m: int, T: int) -> int:
    """Standard NS with symmetric GEMMs, T(3 alpha + 1) n^3 (section "1. Gram Newton-Schulz")."""
    return T * (3 * m * n * n + n ** 3)


def flops_gram_formula(n: int, m: int, T: int) -> int:
    """Naive Gram NS cost T*4n^3 + 3mn^2 - 3n^3 (section "1. Gram Newton-Schulz")."""
    return T * 4 * n ** 3 + 3 * m * n * n - 3 * n ** 3


def flops_restart_formula(n: int, m: int) -> int:
    """Extra cost of one restart, 3(alpha - 1) n^3 (section "1. Gram Newton-Schulz")."""
    return 3 * m * n * n - 3 * n ** 3


# --------------------------------------------------------------------------------------
# Polar factor (Definition 1)
# --------------------------------------------------------------------------------------

def polar_svd(x) -> np.ndarray:
    """polar(X) = U V^T from the thin SVD X = U Sigma V^T (Definition 1)."""
    x = np.asarray(x, dtype=np.float64)
    u, _, vt = np.linalg.svd(x, full_matrices=False)
    return u @ vt


def _coeff_list(coeffs) -> list[tuple[float, float, float]]:
    out = [tuple(float(c) for c in abc) for abc in coeffs]
    for abc in out:
        if len(abc) != 3:
            raise ValueError("each NS step needs three coefficients (a_t, b_t, c_t)")
    return out


def _short_side(x: np.ndarray) -> tuple[np.ndarray, bool]:
    """Return X oriented n x m with n <= m, and whether it was transposed."""
    return (x.T, True) if x.shape[0] > x.shape[1] else (x, False)


# --------------------------------------------------------------------------------------
# Standard quintic Newton-Schulz (section "Standard Newton-Schulz")
# --------------------------------------------------------------------------------------

def newton_schulz(x, coeffs, counter: FlopCounter | None = None) -> np.ndarray:
    """Standard Newton-Schulz approximation of polar(X).

    X_0 = X / ||X||_F, then for each t with coefficients (a_t, b_t, c_t):
        A = X_t X_t^T,  X_{t+1} = a_t X_t + (b_t A + c_t A^2) X_t,
    which is the page's a X + b X X^T X + c (X X^T)^2 X written with A and A^2, the two
    symmetric products the page names. Runs on the short side (tall inputs transposed)."""
    x = np.asarray(x, dtype=np.float64)
    xs, tall = _short_side(x)
    nrm = frobenius(xs)
    if nrm == 0.0:
        return np.zeros_like(x)
    X = xs / nrm
    for a, b, c in _coeff_list(coeffs):
        A = _mm(X, X.T, counter, symmetric=True)
        B = b * A + c * _mm(A, A, counter, symmetric=True)
        X = a * X + _mm(B, X, counter)
    return X.T if tall else X


# --------------------------------------------------------------------------------------
# Gram Newton-Schulz (Theorem 2, naive algorithm, restart, Algorithm 3)
# --------------------------------------------------------------------------------------

def gram_newton_schulz(x, coeffs, restart_before: Iterable[int] = (),
                       counter: FlopCounter | None = None) -> np.ndarray:
    """Gram Newton-Schulz: iterate on the n x n Gram side, then apply Q_T to X.

    Theorem 2 with p_t(x) = a_t x + b_t x^3 + c_t x^5 = x h_t(x^2), h_t(y) = a_t + b_t y
    + c_t y^2, lifted to matrices: R_0 = X_0 X_0^T, Q_0 = I and per iteration
        Z_t = h_t(R_{t-1}),  R_t = R_{t-1} Z_t^2,  Q_t = Q_{t-1} Z_t;  output Q_T X_0.
    ``restart_before`` holds iterations t before which the stabilising restart runs:
    X <- Q X, R <- X X^T, Q <- I (section "Stabilization via Restarting"). Products whose
    result is never used are not formed: Q_1 = Z_1 (Q_0 = I), R_T, and R_{t-1} when a
    restart replaces it -- which is exactly the set the page's FLOP counts price."""
    x = np.asarray(x, dtype=np.float64)
    xs, tall = _short_side(x)
    nrm = frobenius(xs)
    if nrm == 0.0:
        return np.zeros_like(x)
    coeff = _coeff_list(coeffs)
    T = len(coeff)
    restarts = set(int(t) for t in restart_before)
    X = xs / nrm
    n = X.shape[0]
    eye = np.eye(n)
    R = _mm(X, X.T, counter, symmetric=True)
    Q = None                                    # None stands for the identity
    for t, (a, b, c) in enumerate(coeff, start=1):
        if t in restarts and t > 1:
            if Q is not None:
                X = _mm(Q, X, counter)
            R = _mm(X, X.T, counter, symmetric=True)
            Q = None
        Z = a * eye + b * R + c * _mm(R, R, counter, symmetric=True)
        Q = Z if Q is None else _mm(Q, Z, counter, symmetric=True)
        if t < T and (t + 1) not in restarts:
            Z2 = _mm(Z, Z, counter, symmetric=True)
            R = _mm(R, Z2, counter, symmetric=True)
    out = X if Q is None else _mm(Q, X, counter)
    return out.T if tall else out


def orthogonalize(x, coeffs, kind: str = "standard", restart_before: Iterable[int] = (),
                  counter: FlopCounter | None = None) -> np.ndarray:
    if kind == "standard":
        return newton_schulz(x, coeffs, counter)
    if kind == "gram":
        return gram_newton_schulz(x, coeffs, restart_before, counter)
    raise ValueError(f"unknown NS kind {kind!r}")


# --------------------------------------------------------------------------------------
# NorMuon (Eq. 2)
# --------------------------------------------------------------------------------------

def normuon_update(O, v, beta2: float, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """NorMuon per-row normalisation of an orthogonalised update O (Eq. 2).

    v_i <- beta2 v_i + (1 - beta2) (1/m) sum_j O_ij^2,  Ohat_ij = O_ij / (sqrt(v_i) + eps),
    returns (v_new, U) with U = (||O||_F / ||Ohat||_F) Ohat, the step applied as
    W <- W - eta U. Rows are stored rows of W, m their length."""
    O = np.asarray(O, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m = O.shape[1]
    row_sq = np.sum(O * O, axis=1)
    v_new = beta2 * v + (1.0 - beta2) * row_sq / m
    O_hat = O / (np.sqrt(v_new) + eps)[:, None]
    n_o, n_hat = frobenius(O), frobenius(O_hat)
    ratio = n_o / n_hat if n_hat > 0.0 else 0.0
    return v_new, ratio * O_hat


# --------------------------------------------------------------------------------------
# Muon step (Eq. 1) with the optional NorMuon variant (Eq. 2)
# --------------------------------------------------------------------------------------

def muon_step(W, M, G, *, mu: float, lr: float, coeffs, kind: str = "standard",
              restart_before: Iterable[int] = (), normuon: bool = False, v=None,
              beta2: float = 0.95, eps: float = 1e-8, storage: str = "bf16",
              counter: FlopCounter | None = None) -> dict:
    """One Muon step (Eq. 1): M <- mu M + G; W <- W - eta polar(M), polar by NS.

    With ``normuon`` the update is NorMuon's (Eq. 2). W is rounded once, to ``storage``,
    from the exact float64 value W + update; M and v are returned in float64."""
    W = np.asarray(W, dtype=np.float64)
    M_new = mu * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    O = orthogonalize(M_new, coeffs, kind, restart_before, counter)
    v_new = None
    U = O
    if normuon:
        v0 = np.zeros(W.shape[0]) if v is None else v
        v_new, U = normuon_update(O, v0, beta2, eps)
    W_exact = W - lr * U
    return {"W": round_to_storage(W_exact, storage), "W_exact": W_exact, "M": M_new,
            "v": v_new, "O": O, "U": U}


# --------------------------------------------------------------------------------------
# Dion3 fractional row selection (Algorithm 4) and the learning-rate transfer rule
# --------------------------------------------------------------------------------------

def rows_for_fraction(f: float, n: int) -> int:
    """k = ceil(f n) selected rows, f in (0, 1] (Algorithm 4, Selection)."""
    if not (0.0 < f <= 1.0):
        raise ValueError("row fraction must lie in (0, 1]")
    return max(1, min(n, int(math.ceil(f * n))))


def transfer_lr(lr: float, f: float) -> float:
    """eta' = eta / sqrt(f) (section "Model Quality", learning-rate transfer rule)."""
    return lr / math.sqrt(f)


def select_rows(M, k: int) -> np.ndarray:
    """Indices of the k rows of M with the largest l1 norm, largest first; equal norms
    are ordered by the lower row index (Algorithm 4, Selection)."""
    M = np.asarray(M, dtype=np.float64)
    l1 = np.sum(np.abs(M), axis=1)
    order = np.lexsort((np.arange(M.shape[0]), -l1))
    return order[:k].astype(np.int64)


def dion3_step(W, M, G, *, mu: float, lr: float, f: float, coeffs, kind: str = "gram",
               restart_before: Iterable[int] = (), normuon: bool = False, v=None,
               beta2: float = 0.95, eps: float = 1e-8, storage: str = "bf16",
               rows: Sequence[int] | None = None,
               counter: FlopCounter | None = None) -> dict:
    """One Dion3 step on a single weight matrix (Algorithm 4).

    M <- M + G; S = top-k rows by l1 (k = ceil(f n)); O = polar(M[S, :]) by (Gram) NS;
    W[S, :] <- W[S, :] - eta U with U = O or its NorMuon form over the selected rows;
    error feedback M <- mu Mhat + (M - Mhat), i.e. only rows in S are decayed by mu.
    ``rows`` overrides the selection (used to re-run a step on another side's S)."""
    W = np.asarray(W, dtype=np.float64).copy()
    M_new = np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    n = M_new.shape[0]
    k = rows_for_fraction(f, n)
    S = select_rows(M_new, k) if rows is None else np.asarray(rows, dtype=np.int64)
    O = orthogonalize(M_new[S, :], coeffs, kind, restart_before, counter)
    v_new = None if v is None else np.asarray(v, dtype=np.float64).copy()
    U = O
    if normuon:
        if v_new is None:
            v_new = np.zeros(n)
        v_sel, U = normuon_update(O, v_new[S], beta2, eps)
        v_new[S] = v_sel
    W_exact = W.copy()
    W_exact[S, :] = W[S, :] - lr * U
    M_out = M_new.copy()
    M_out[S, :] = mu * M_new[S, :]
    return {"W": round_to_storage(W_exact, storage), "W_exact": W_exact, "M": M_out,
            "v": v_new, "O": O, "U": U, "S": S, "M_selected": M_new[S, :]}
