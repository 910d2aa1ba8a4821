"""The five benchmark/parity workloads, as data.

Shapes, dtypes and hyperparameters of each workload; the coefficient triple is a stated
parameter of the quintic Newton-Schulz iteration, used for every iteration t.
"""
from __future__ import annotations

from dataclasses import dataclass, field

QUINTIC = (3.4445, -4.7750, 2.0315)
# The odd quintic with p(1) = 1, p'(1) = p''(1) = 0: p(x) = (15 x - 10 x^3 + 3 x^5) / 8, whose
# iteration converges to the polar factor (singular values -> 1) once they are near 1.
CONVERGENT = (15.0 / 8.0, -10.0 / 8.0, 3.0 / 8.0)


@dataclass(frozen=True)
class MatrixSpec:
    rows: int
    cols: int
    count: int = 1          # how many matrices of this shape (one shape group)


@dataclass(frozen=True)
class Workload:
    index: int              # 1-based workload number
    name: str
    storage: str            # 'f32' or 'bf16'
    groups: tuple           # tuple[MatrixSpec]
    dist: str               # gradient distribution, see synthetic.DISTRIBUTIONS
    mu: float = 0.95
    lr: float = 0.02
    T: int = 5
    coeffs: tuple = QUINTIC      # one (a, b, c) for every t, or a tuple of T of them
    kind: str = "standard"  # 'standard' or 'gram'
    restart_before: tuple = ()
    normuon: bool = False
    beta2: float = 0.95
    eps: float = 1e-8
    row_fraction: float = 1.0
    steps: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def n_matrices(self) -> int:
        return sum(g.count for g in self.groups)

    def matrices(self):
        """(index, rows, cols) for every matrix, in group order."""
        out, i = [], 0
        for g in self.groups:
            for _ in range(g.count):
                out.append((i, g.rows, g.cols))
                i += 1
        return out

    def coeff_table(self):
        if isinstance(self.coeffs[0], (tuple, list)):
            assert len(self.coeffs) == self.T
            return [tuple(c) for c in self.coeffs]
        return [self.coeffs] * self.T


WORKLOADS = {
    1: Workload(1, "fp32 256x1024 single matrix", "f32", (MatrixSpec(256, 1024),), "normal",
                steps=1),
    2: Workload(2, "4 x 4096x4096 bf16 (attention-like)", "bf16", (MatrixSpec(4096, 4096, 4),),
                "lowrank", steps=2),
    3: Workload(3, "4096x16384 bf16 MLP (alpha=4)", "bf16", (MatrixSpec(4096, 16384),),
                "student_t", steps=1, extra={"cross_check_gram": True}),
    4: Workload(4, "3B-like layer set: 28 x {4x3072^2, 2x3072x8192, 1x8192x3072} bf16", "bf16",
                (MatrixSpec(3072, 3072, 4 * 28), MatrixSpec(3072, 8192, 2 * 28),
                 MatrixSpec(8192, 3072, 1 * 28)),
                "normal", normuon=True, steps=1),
    5: Workload(5, "14B-scale MLP 5120x13824 bf16, Dion3 f=1/4, 10 steps", "bf16",
                (MatrixSpec(5120, 13824),), "student_t", kind="gram", restart_before=(3,),
                normuon=True, row_fraction=0.25, lr=0.04, steps=10),
    # high aspect ratio, as in fine-grained MoE experts: the regime where the Gram
    # reformulation saves the most (Gram NS + restart vs standard NS: 2.02x fewer FLOPs)
    6: Workload(6, "MoE experts: 32 x 1024x8192 bf16 (alpha=8)", "bf16",
                (MatrixSpec(1024, 8192, 32),), "normal", kind="gram", restart_before=(3,),
                steps=1, extra={"cross_check_standard": True}),
    # a per-iteration coefficient schedule: four quintic steps, then two convergent ones
    7: Workload(7, "coefficient schedule: 4 x 2048x8192 bf16, T=6 (4 quintic + 2 convergent)",
                "bf16", (MatrixSpec(2048, 8192, 4),), "student_t", T=6,
                coeffs=(QUINTIC,) * 4 + (CONVERGENT,) * 2, steps=1),
}
