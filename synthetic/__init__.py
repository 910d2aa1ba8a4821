"""Seeded synthetic inputs for the Muon-family optimizer step.

This module is the only code shared by the HIP path's tests/benchmark and the fp64 oracle.
It holds no arithmetic of the method: it draws random gradients, weights and states from
fixed seeds and encodes them in the stored formats (float32 or bfloat16 bit patterns).
Both sides then consume the identical stored bits.

Seeds: ``numpy.random.default_rng([tag, config, step, index])`` (PCG64 seeded through
SeedSequence with a list of integers), so every matrix of every step of every workload is
reproducible on any machine.
"""
from __future__ import annotations

import numpy as np

from .configs import WORKLOADS, Workload, MatrixSpec  # noqa: F401

_TAG_GRAD = 0x6D6E73          # distinct streams for gradients, weights and states
_TAG_WEIGHT = 0x77
_TAG_STATE = 0x5E


def rng_for(tag: int, config: int, step: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(tag), int(config), int(step), int(index)])


def encode(x, storage: str) -> np.ndarray:
    """Encode values in a stored format.

    'f32'  -> float32 array (IEEE round-to-nearest-even from float64).
    'bf16' -> uint16 bfloat16 bit patterns: float32 first, then the upper 16 bits rounded
              to nearest even (finite inputs only; the generators draw finite values)."""
    f32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if storage == "f32":
        return f32
    if storage == "bf16":
        u = f32.view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown storage {storage!r}")


def decode(stored, storage: str) -> np.ndarray:
    """Stored format -> float32 values (exact)."""
    if storage == "f32":
        return np.asarray(stored, dtype=np.float32)
    if storage == "bf16":
        u = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32)
    raise ValueError(f"unknown storage {storage!r}")


# ---- value distributions ------------------------------------------------------------

def normal(rows: int, cols: int, rng: np.random.Generator, std: float = 1.0) -> np.ndarray:
    return rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)


def lowrank_plus_noise(rows: int, cols: int, rng: np.random.Generator, rank: int = 64,
                       noise_std: float = 0.1) -> np.ndarray:
    """(A B)/sqrt(rank) + noise_std * N: a rank-``rank`` part with unit-variance entries
    plus i.i.d. Gaussian noise (attention-projection-like gradients)."""
    a = rng.standard_normal((rows, rank))
    b = rng.standard_normal((rank, cols))
    low = (a @ b) / np.sqrt(rank)
    return (low + noise_std * rng.standard_normal((rows, cols))).astype(np.float32)


def student_t_unit_rms(rows: int, cols: int, rng: np.random.Generator,
                       nu: float = 3.0) -> np.ndarray:
    """Heavy-tailed Student-t(nu) entries scaled to unit empirical RMS."""
    t = rng.standard_t(nu, size=(rows, cols))
    rms = np.sqrt(np.mean(t * t))
    return (t / rms).astype(np.float32)


DISTRIBUTIONS = {
    "normal": normal,
    "lowrank": lowrank_plus_noise,
    "student_t": student_t_unit_rms,
}


def gradient(dist: str, rows: int, cols: int, storage: str, config: int, step: int,
             index: int) -> np.ndarray:
    """A seeded synthetic gradient in its stored format."""
    rng = rng_for(_TAG_GRAD, config, step, index)
    return encode(DISTRIBUTIONS[dist](rows, cols, rng), storage)


def weight(rows: int, cols: int, storage: str, config: int, index: int,
           zero: bool = True) -> np.ndarray:
    """Initial weights: zero, or N(0, 1/cols) entries."""
    if zero:
        return encode(np.zeros((rows, cols), dtype=np.float32), storage)
    rng = rng_for(_TAG_WEIGHT, config, 0, index)
    return encode(normal(rows, cols, rng, std=1.0 / np.sqrt(cols)), storage)


def state(rows: int, cols: int, config: int, index: int, scale: float = 0.0) -> np.ndarray:
    """Initial float32 momentum: zero, or scale * N(0, 1)."""
    if scale == 0.0:
        return np.zeros((rows, cols), dtype=np.float32)
    rng = rng_for(_TAG_STATE, config, 0, index)
    return normal(rows, cols, rng, std=scale)
