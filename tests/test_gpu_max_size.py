"""The largest iterate the library accepts (rows and cols padded to 256 plus the 256-element
row pitch, under 2 GiB in both layouts), with ragged padding, checked against the oracle
through a closed form that holds at any size: for a rectangular-diagonal input, Newton-Schulz
keeps the singular vectors, so the output is rectangular-diagonal with entries phi(s_i/||s||)
(phi = the composed polynomials), and every off-diagonal entry stays exactly zero (products of
diagonal matrices never create non-zeros). phi at each distinct value comes from the oracle,
run on a 2x2 diagonal matrix with the same normalised entry."""
import numpy as np
import pytest
import torch

import oracle
import muon_newton_schulz_amd as mns
from helpers import TOL

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)
VALUES = np.array([1.0, 2.0, 0.5, 3.0, 0.25, 1.5, 4.0, 0.75])   # exact in bfloat16


def _say(*a):
    print(*a, flush=True)


def _phi_from_oracle(t, coeffs):
    """phi(t) for 0 < t < 1: the oracle on diag(t, sqrt(1 - t^2)) (Frobenius norm 1)."""
    return oracle.newton_schulz(np.diag([t, np.sqrt(1.0 - t * t)]), coeffs)[0, 0]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,tall", [("standard", False), ("gram", False), ("standard", True)])
def test_max_size_rectangular_diagonal(kind, tall):
    n, m = 16380, 64500          # padded: 16384 x 64512, the largest m for this n
    _say("case", kind, "tall" if tall else "wide", n, m)
    coeffs = [QUINTIC] * 5
    s = VALUES[np.arange(n) % len(VALUES)]
    t = VALUES / np.sqrt(np.sum(s * s))
    want_k = np.array([_phi_from_oracle(x, coeffs) for x in t])
    want = want_k[np.arange(n) % len(VALUES)]
    shape = (m, n) if tall else (n, m)
    X = torch.zeros(*shape, dtype=torch.bfloat16, device="cuda")
    X.diagonal().copy_(torch.from_numpy(s).to(torch.bfloat16))
    if kind == "standard":
        O = mns.ns_orthogonalize(X, coeffs)
    else:
        O = mns.gram_ns_orthogonalize(X, coeffs, restart_before=(3,))
    torch.cuda.synchronize()
    got = O.diagonal().double().cpu().numpy()
    nonzero = int((O != 0).sum().item())
    err = np.linalg.norm(got - want) / np.linalg.norm(want)
    _say(f"  diagonal rel err {err:.2e}; non-zeros {nonzero} (diagonal length {n})")
    assert nonzero == n
    assert err < TOL["bf16"]
