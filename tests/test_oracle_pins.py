"""Pins for the fp64 oracle, against what the page "Dion3: Full-stack orthogonal updates"
and the mathematics fix. Each test reaches the expected value by a different route than
the oracle's own code: SVD closed forms, a textbook special case, Theorem 2's equivalence,
the page's printed FLOP formulas, a hand-worked fixture, brute force, invariants.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from synthetic import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
QUINTIC = (3.4445, -4.7750, 2.0315)


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b))


def _scalar_map(coeffs, s):
    """p_T o ... o p_1 on scalars, p_t(x) = a x + b x^3 + c x^5 (section 'Standard
    Newton-Schulz': each iteration maps singular values by its odd quintic)."""
    s = np.asarray(s, dtype=np.float64)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def _closed_form(x, coeffs):
    """NS_T(X) = U diag(phi(sigma / ||X||_F)) V^T: NS keeps singular vectors and maps
    singular values through the composed polynomial."""
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    phi = _scalar_map(coeffs, s / np.sqrt(np.sum(s * s)))
    return (u * phi) @ vt


# ---- storage encodings ---------------------------------------------------------------

def test_bf16_rounding_fixed_points():
    cases = {
        1.0: 0x3F80, -2.0: 0xC000, 0.0: 0x0000,
        1.0 + 2.0 ** -8: 0x3F80,            # halfway, ties to even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # halfway, ties to even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above halfway rounds up
        float.fromhex("0x1.fep127"): 0x7F7F,    # largest finite
        float.fromhex("0x1.ffp127"): 0x7F80,    # halfway to 2^128 -> even -> inf
        2.0 ** -133: 0x0001,                 # smallest subnormal
        2.0 ** -134: 0x0000,                 # halfway to zero, ties to even (zero)
        3 * 2.0 ** -134: 0x0002,             # 1.5 ulp -> 2 (even)
    }
    for x, bits in cases.items():
        assert int(oracle.f64_to_bf16_bits(np.array([x]))[0]) == bits, (x, hex(bits))


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-60, 60, 200_000))).astype(np.float32)
    ours = oracle.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_is_exact_inverse():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = oracle.f64_to_bf16_bits(vals[finite])
    assert np.array_equal(back, bits[finite])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(vals[finite], ref[finite])


# ---- polar factor (Definition 1) -----------------------------------------------------

@pytest.mark.parametrize("shape", [(6, 15), (15, 6), (9, 9)])
def test_polar_svd_satisfies_polar_decomposition(shape):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(shape)
    p = oracle.polar_svd(x)
    n = min(shape)
    # orthonormal short side
    g = p @ p.T if shape[0] <= shape[1] else p.T @ p
    assert np.allclose(g, np.eye(n), atol=1e-12)
    # X = H P (wide) or P H (tall) with H symmetric positive definite
    h = x @ p.T if shape[0] <= shape[1] else p.T @ x
    assert np.allclose(h, h.T, atol=1e-12)
    assert np.linalg.eigvalsh((h + h.T) / 2).min() > 0
    recon = h @ p if shape[0] <= shape[1] else p @ h
    assert np.allclose(recon, x, atol=1e-12)


# ---- standard Newton-Schulz -----------------------------------------------------------

@pytest.mark.parametrize("shape", [(8, 20), (20, 8), (16, 16), (5, 40), (1, 12)])
def test_newton_schulz_matches_svd_closed_form(shape):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(shape)
    coeffs = [QUINTIC] * 5
    assert _rel(oracle.newton_schulz(x, coeffs), _closed_form(x, coeffs)) < 1e-12


def test_newton_schulz_uses_coefficients_per_iteration():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, 30))
    coeffs = [(3.0, -3.2, 1.2), (2.5, -2.0, 0.6), (1.9, -1.3, 0.4), (1.5, -0.5, 0.0)]
    assert _rel(oracle.newton_schulz(x, coeffs), _closed_form(x, coeffs)) < 1e-12
    # reversing the schedule changes the result: iteration t must use its own (a_t, b_t, c_t)
    assert _rel(oracle.newton_schulz(x, coeffs[::-1]), _closed_form(x, coeffs)) > 1e-3


def test_newton_schulz_rank_deficient_closed_form():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((12, 4)) @ rng.standard_normal((4, 30))
    coeffs = [QUINTIC] * 5
    assert _rel(oracle.newton_schulz(x, coeffs), _closed_form(x, coeffs)) < 1e-10


def test_textbook_cubic_converges_to_polar():
    """(a, b, c) = (1.5, -0.5, 0) is the classical cubic Newton-Schulz iteration for the
    polar factor; with singular values in (0, 1] it converges to U V^T (Definition 1)."""
    rng = np.random.default_rng(6)
    for shape in [(16, 40), (40, 16), (24, 24)]:
        x = rng.standard_normal(shape)
        out = oracle.newton_schulz(x, [(1.5, -0.5, 0.0)] * 40)
        assert _rel(out, oracle.polar_svd(x)) < 1e-12


def test_singular_values_within_scalar_map_band():
    """Quintic NS pushes singular values towards 1: for the 256x1024 Gaussian workload
    the output singular values lie in phi([s_min, s_max]) and are far less spread."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((256, 1024))
    coeffs = [QUINTIC] * 5
    out = oracle.newton_schulz(x, coeffs)
    s_in = np.linalg.svd(x, compute_uv=False)
    s_out = np.linalg.svd(out, compute_uv=False)
    grid = np.linspace(s_in.min(), s_in.max(), 20001) / np.sqrt(np.sum(s_in ** 2))
    band = _scalar_map(coeffs, grid)
    assert s_out.min() >= band.min() - 1e-12 and s_out.max() <= band.max() + 1e-12
    assert s_out.max() / s_out.min() < 1.7 < s_in.max() / s_in.min()
    assert 0.6 < s_out.min() and s_out.max() < 1.2


def test_convergent_quintic_is_second_order_at_one():
    """The schedule workload's last polynomial, (15 x - 10 x^3 + 3 x^5) / 8, fixes 1 with
    zero first and second derivative (so iterating it converges to the polar factor)."""
    a, b, c = synthetic.configs.CONVERGENT
    assert a + b + c == 1.0
    assert a + 3 * b + 5 * c == 0.0
    assert 6 * b + 20 * c == 0.0


@pytest.mark.parametrize("shape,seed", [((64, 256), 1), ((128, 512), 2), ((400, 48), 3)])
def test_coefficient_schedule_reaches_polar(shape, seed):
    """Four quintic steps then two convergent ones: the closed form with per-iteration
    coefficients holds, and the output is the polar factor to ~1e-4 (the plain quintic
    schedule stays ~0.2 away: its fixed point is not 1)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    sched = WORKLOADS[7].coeff_table()
    out = oracle.newton_schulz(x, sched)
    assert _rel(out, _closed_form(x, sched)) < 1e-12
    assert _rel(out, oracle.polar_svd(x)) < 1e-3
    assert _rel(oracle.newton_schulz(x, [QUINTIC] * 6), oracle.polar_svd(x)) > 0.1
    s = np.linalg.svd(out, compute_uv=False)
    assert 0.999 < s.min() and s.max() < 1.0 + 1e-5


def test_permutation_equivariance():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((12, 40))
    perm = rng.permutation(12)
    coeffs = [QUINTIC] * 5
    for fn in (oracle.newton_schulz,
               lambda z, c: oracle.gram_newton_schulz(z, c, restart_before=(3,))):
        assert _rel(fn(x[perm], coeffs), fn(x, coeffs)[perm]) < 1e-12


def test_zero_input_gives_zero():
    z = np.zeros((4, 9))
    assert not oracle.newton_schulz(z, [QUINTIC] * 5).any()
    assert not oracle.gram_newton_schulz(z, [QUINTIC] * 5, restart_before=(3,)).any()


# ---- Gram Newton-Schulz (Theorem 2, restart) ------------------------------------------

@pytest.mark.parametrize("shape", [(24, 96), (96, 24), (32, 32), (7, 50)])
@pytest.mark.parametrize("restarts", [(), (3,), (2, 4)])
def test_gram_ns_equals_standard_ns(shape, restarts):
    rng = np.random.default_rng(9)
    x = rng.standard_normal(shape)
    coeffs = [QUINTIC] * 5
    std = oracle.newton_schulz(x, coeffs)
    gram = oracle.gram_newton_schulz(x, coeffs, restart_before=restarts)
    assert _rel(gram, std) < 1e-11


def test_gram_ns_on_diagonal_input_is_scalar_map():
    """Theorem 2 on scalars: for X = [diag(s) | 0] the Gram recurrence acts entrywise and
    must return diag(p_T o ... o p_1 (s / ||s||))."""
    s = np.array([3.0, 1.0, 0.5, 0.25, 0.01])
    x = np.zeros((5, 11))
    x[np.arange(5), np.arange(5)] = s
    coeffs = [(3.0, -3.2, 1.2), QUINTIC, (2.0, -1.5, 0.5), QUINTIC]
    for restarts in [(), (3,)]:
        out = oracle.gram_newton_schulz(x, coeffs, restart_before=restarts)
        want = np.zeros_like(x)
        want[np.arange(5), np.arange(5)] = _scalar_map(coeffs, s / np.linalg.norm(s))
        assert np.allclose(out, want, rtol=0, atol=1e-13)


# ---- FLOP counts (page formulas) ------------------------------------------------------

@pytest.mark.parametrize("n,m,T", [(64, 256, 5), (32, 32, 5), (16, 128, 3), (8, 80, 7)])
def test_flop_counter_reproduces_page_formulas(n, m, T):
    rng = np.random.default_rng(10)
    x = rng.standard_normal((n, m))
    coeffs = [QUINTIC] * T
    alpha = m / n
    c = oracle.FlopCounter()
    oracle.newton_schulz(x, coeffs, counter=c)
    assert c.dense == oracle.flops_standard_formula(n, m, T)
    assert c.dense == round(2 * T * (2 * alpha + 1) * n ** 3)
    assert c.algorithmic == oracle.flops_standard_symmetric_formula(n, m, T)
    assert c.algorithmic == round(T * (3 * alpha + 1) * n ** 3)
    assert len(c.products) == 3 * T
    g = oracle.FlopCounter()
    oracle.gram_newton_schulz(x, coeffs, counter=g)
    assert g.algorithmic == oracle.flops_gram_formula(n, m, T)
    assert g.algorithmic == round((4 * T + 3 * alpha - 3) * n ** 3)
    r = oracle.FlopCounter()
    oracle.gram_newton_schulz(x, coeffs, restart_before=(3,), counter=r)
    assert r.algorithmic - g.algorithmic == oracle.flops_restart_formula(n, m)
    assert r.algorithmic - g.algorithmic == round(3 * (alpha - 1) * n ** 3)


def test_fifteen_gemms_and_55_percent_saving():
    """T = 5 standard NS is (20 alpha + 10) n^3 over 15 GEMMs; at alpha = 4 Gram NS saves
    55% of the FLOPs of standard NS with symmetric GEMMs."""
    n, m, T = 16, 64, 5
    c = oracle.FlopCounter()
    oracle.newton_schulz(np.random.default_rng(11).standard_normal((n, m)), [QUINTIC] * T, c)
    assert len(c.products) == 15 and c.dense == (20 * 4 + 10) * n ** 3
    saving = 1 - oracle.flops_gram_formula(n, m, T) / oracle.flops_standard_symmetric_formula(n, m, T)
    assert round(100 * saving) == 55
    assert abs(saving - (1 - 29 / 65)) < 1e-15


# ---- NorMuon (Eq. 2) ------------------------------------------------------------------

def test_normuon_hand_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "normuon_worked.json")))
    v, u = oracle.normuon_update(np.array(d["O"]), np.array(d["v0"]), d["beta2"], d["eps"])
    assert np.allclose(v, d["expected_v"], rtol=0, atol=1e-15)
    assert np.allclose(u, d["expected_update"], rtol=1e-15)
    w = np.array(d["W0"]) - d["lr"] * u
    assert np.allclose(w, d["expected_W"], rtol=1e-15)


def test_normuon_preserves_update_norm():
    rng = np.random.default_rng(12)
    o = rng.standard_normal((20, 50)) * rng.uniform(0.1, 3, (20, 1))
    v0 = rng.uniform(0, 2, 20)
    _, u = oracle.normuon_update(o, v0, 0.95, 1e-8)
    assert abs(np.linalg.norm(u) - np.linalg.norm(o)) < 1e-12 * np.linalg.norm(o)


def test_normuon_equal_row_norms_is_plain_muon():
    """An exact polar factor of a wide full-rank matrix has orthonormal rows, so every
    row has the same norm and NorMuon's update equals O."""
    rng = np.random.default_rng(13)
    o = oracle.polar_svd(rng.standard_normal((12, 40)))
    _, u = oracle.normuon_update(o, np.zeros(12), 0.95, 1e-8)
    assert np.allclose(u, o, rtol=0, atol=1e-13)


def test_normuon_beta2_zero_is_row_rms_normalisation():
    rng = np.random.default_rng(14)
    o = rng.standard_normal((6, 10)) * np.arange(1, 7)[:, None]
    v, u = oracle.normuon_update(o, np.full(6, 5.0), 0.0, 0.0)
    rms = np.sqrt(np.mean(o ** 2, axis=1))
    assert np.allclose(v, rms ** 2, rtol=1e-14)
    o_hat = o / rms[:, None]
    assert np.allclose(u, o_hat * np.linalg.norm(o) / np.linalg.norm(o_hat), rtol=1e-13)


def test_normuon_zero_update():
    v, u = oracle.normuon_update(np.zeros((3, 4)), np.array([1.0, 2.0, 0.0]), 0.5, 1e-8)
    assert np.allclose(v, [0.5, 1.0, 0.0]) and not u.any()


# ---- Muon step (Eq. 1) ----------------------------------------------------------------

def test_muon_step_composition():
    rng = np.random.default_rng(15)
    W = rng.standard_normal((6, 14))
    M = rng.standard_normal((6, 14))
    G = rng.standard_normal((6, 14))
    coeffs = [QUINTIC] * 5
    out = oracle.muon_step(W, M, G, mu=0.9, lr=0.05, coeffs=coeffs, storage="f32")
    m1 = 0.9 * M + G
    assert np.array_equal(out["M"], m1)
    assert np.allclose(out["W_exact"], W - 0.05 * _closed_form(m1, coeffs), rtol=0, atol=1e-13)
    assert np.array_equal(out["W"], out["W_exact"].astype(np.float32).astype(np.float64))


def test_muon_step_gram_kind_matches_standard():
    rng = np.random.default_rng(16)
    W, M, G = (rng.standard_normal((10, 30)) for _ in range(3))
    kw = dict(mu=0.95, lr=0.02, coeffs=[QUINTIC] * 5, storage="f32", normuon=True,
              v=np.zeros(10))
    a = oracle.muon_step(W, M, G, kind="standard", **kw)
    b = oracle.muon_step(W, M, G, kind="gram", restart_before=(3,), **kw)
    assert _rel(b["W_exact"] - W, a["W_exact"] - W) < 1e-11
    assert _rel(b["v"], a["v"]) < 1e-11


# ---- Dion3 (Algorithm 4) and the learning-rate transfer rule --------------------------

def test_select_rows_brute_force():
    rng = np.random.default_rng(17)
    for n, k in [(7, 3), (8, 1), (6, 6), (9, 4)]:
        M = rng.standard_normal((n, 5))
        l1 = np.abs(M).sum(axis=1)
        best = max(itertools.combinations(range(n), k), key=lambda s: sum(l1[list(s)]))
        got = oracle.select_rows(M, k)
        assert sorted(got.tolist()) == sorted(best)
        assert np.all(np.diff(l1[got]) <= 0)          # largest first


def test_select_rows_ties_prefer_lower_index():
    base = np.array([1.0, -2.0, 3.0])
    M = np.stack([base * 0.5, base[::-1], -base, base[[1, 2, 0]], base * 2.0])
    # rows 1, 2, 3 have equal l1 norm (6); row 4 has 12; row 0 has 3
    assert oracle.select_rows(M, 3).tolist() == [4, 1, 2]
    assert oracle.select_rows(M, 4).tolist() == [4, 1, 2, 3]


def test_select_rows_nonfinite_norms():
    """Non-finite norms (a reading of Algorithm 4, which is silent on them): an infinite l1 norm
    ranks above every finite one, a NaN norm below every number, and equal keys, NaN ones
    included, go to the lower row index."""
    M = np.ones((6, 4))
    M[1, 2] = np.nan
    M[4, 0] = np.nan
    M[3, 1] = np.inf
    M[5] *= 2.0
    # l1: 4, NaN, 4, inf, NaN, 8
    assert oracle.select_rows(M, 6).tolist() == [3, 5, 0, 2, 1, 4]
    assert oracle.select_rows(M, 4).tolist() == [3, 5, 0, 2]


def test_rows_for_fraction():
    assert oracle.rows_for_fraction(0.25, 5120) == 1280
    assert oracle.rows_for_fraction(1 / 3, 10) == 4
    assert oracle.rows_for_fraction(1.0, 7) == 7
    assert oracle.rows_for_fraction(1e-9, 7) == 1
    for bad in (0.0, -0.5, 1.5):
        with pytest.raises(ValueError):
            oracle.rows_for_fraction(bad, 10)


def test_dion3_full_fraction_is_muon():
    rng = np.random.default_rng(18)
    W, M, G = (rng.standard_normal((9, 25)) for _ in range(3))
    v = rng.uniform(0, 1, 9)
    kw = dict(mu=0.9, lr=0.03, coeffs=[QUINTIC] * 5, kind="gram", restart_before=(3,),
              normuon=True, v=v, storage="f32")
    # Dion3 keeps its momentum already decayed (error feedback decays after the step), so
    # the Dion3 state that matches a Muon state M is mu * M: both then orthogonalise
    # mu M + G, and the new Dion3 state is mu times the new Muon state.
    d = oracle.dion3_step(W, 0.9 * M, G, f=1.0, **kw)
    m = oracle.muon_step(W, M, G, **kw)
    assert np.allclose(d["W_exact"], m["W_exact"], rtol=0, atol=1e-13)
    assert np.allclose(d["M"], 0.9 * m["M"], rtol=0, atol=1e-14)
    assert np.allclose(d["v"], m["v"], rtol=1e-13)
    assert sorted(d["S"].tolist()) == list(range(9))


def test_dion3_error_feedback_and_row_restriction():
    rng = np.random.default_rng(19)
    W, M, G = (rng.standard_normal((10, 20)) for _ in range(3))
    v = rng.uniform(0, 1, 10)
    d = oracle.dion3_step(W, M, G, mu=0.8, lr=0.1, f=0.5, coeffs=[QUINTIC] * 5,
                          restart_before=(3,), normuon=True, v=v, storage="f32")
    S = d["S"]
    rest = np.setdiff1d(np.arange(10), S)
    assert len(S) == 5
    assert np.array_equal(d["M"][S], 0.8 * (M + G)[S])
    assert np.array_equal(d["M"][rest], (M + G)[rest])      # residual rows keep full weight
    assert np.array_equal(d["W_exact"][rest], W[rest])      # only selected rows move
    assert np.array_equal(d["v"][rest], v[rest])
    assert not np.allclose(d["W_exact"][S], W[S])


def test_lr_transfer_rule_matches_norms():
    """||eta polar(M)||_F = eta sqrt(n) for Muon and eta' sqrt(f n) for Dion3, so
    eta' = eta / sqrt(f) equalises the update norms (section 'Model Quality')."""
    rng = np.random.default_rng(20)
    n, m, f, lr = 16, 48, 0.25, 0.02
    M = rng.standard_normal((n, m))
    k = oracle.rows_for_fraction(f, n)
    S = oracle.select_rows(M, k)
    full = np.linalg.norm(lr * oracle.polar_svd(M))
    part = np.linalg.norm(oracle.transfer_lr(lr, f) * oracle.polar_svd(M[S]))
    assert abs(full - lr * math.sqrt(n)) < 1e-14 and abs(part - full) < 1e-14
    assert abs(oracle.transfer_lr(0.02, WORKLOADS[5].row_fraction) - WORKLOADS[5].lr) < 1e-15


def test_dion3_uses_given_rows():
    rng = np.random.default_rng(21)
    W, M, G = (rng.standard_normal((8, 20)) for _ in range(3))
    rows = [5, 0, 3, 7]
    d = oracle.dion3_step(W, M, G, mu=0.9, lr=0.1, f=0.5, coeffs=[QUINTIC] * 5, rows=rows,
                          storage="f32")
    assert d["S"].tolist() == rows
    want = W[rows] - 0.1 * _closed_form((M + G)[rows], [QUINTIC] * 5)
    assert np.allclose(d["W_exact"][rows], want, rtol=0, atol=1e-13)
