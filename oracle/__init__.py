"""Plain fp64 CPU oracle for the Muon / Newton-Schulz / Gram Newton-Schulz / NorMuon /
Dion3 optimizer step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may call it. It shares
no code with the HIP library (no kernels, headers, helpers or constants); the only thing
both sides consume is the seeded input generator in ``synthetic/``, which holds none of
the method's arithmetic.

Every function follows the page "Dion3: Full-stack orthogonal updates" (arXiv 2608.11612)
and cites the section, equation, theorem or algorithm it implements. All arithmetic is
NumPy float64; library matrix products are used as single steps, with no blocking,
fusion or reordering beyond what the page's own algorithm states.

Pinning status: every public function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, textbook special cases, invariants, hand-worked fixtures or brute
force; none is "parity unpinned".
"""
from .muon import (  # noqa: F401
    FlopCounter,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    round_to_storage,
    frobenius,
    polar_svd,
    newton_schulz,
    gram_newton_schulz,
    orthogonalize,
    normuon_update,
    muon_step,
    select_rows,
    dion3_step,
    rows_for_fraction,
    transfer_lr,
    flops_standard_formula,
    flops_standard_symmetric_formula,
    flops_gram_formula,
    flops_restart_formula,
)
