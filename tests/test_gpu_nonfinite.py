"""Non-finite gradients. A NaN in one matrix of a batched step stays in that matrix: the other
matrices of the same launches come out bit-identical to a step without it, and the matrix
itself ends as the fp64 oracle has it (M NaN only where G is, W and v NaN throughout, as
M / ||M||_F is). A NaN in Dion3's gradient ranks its row below every other (a reading of
Algorithm 4, pinned in the oracle's tests): the row is never selected and the step matches
the oracle's."""
import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as mns
import oracle
import synthetic
from helpers import TOL, check_weight, rel, stored_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)
BF16_NAN = 0x7FC0
HP = dict(mu=0.9, lr=0.05, coeffs=[QUINTIC] * 5, normuon=True, beta2=0.9, eps=1e-8)


def _say(*a):
    print(*a, flush=True)


def _nan_aware(gpu, ref, tol, what):
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(gpu), nan), what
    if (~nan).any():
        assert rel(gpu[~nan], ref[~nan]) < tol, what


def test_nan_gradient_stays_in_its_matrix():
    _say("case NaN in matrix 1 of 3 x 300x700, standard NS + NorMuon")
    shapes = [(300, 700)] * 3
    W0 = [synthetic.weight(r, c, "bf16", 980, i) for i, (r, c) in enumerate(shapes)]
    M0 = [synthetic.state(r, c, 981, i, scale=0.5) for i, (r, c) in enumerate(shapes)]
    v0 = [np.abs(synthetic.state(r, 1, 982, i, scale=0.01)).reshape(r).astype(np.float32)
          for i, (r, c) in enumerate(shapes)]
    G = [synthetic.gradient("student_t", r, c, "bf16", 983, 0, i) for i, (r, c) in enumerate(shapes)]
    G_nan = [g.copy() for g in G]
    G_nan[1][5, 7] = BF16_NAN

    def run(grads):
        W = [to_device(w, "bf16") for w in W0]
        M = [torch.from_numpy(m).cuda() for m in M0]
        v = [torch.from_numpy(x).cuda() for x in v0]
        mns.muon_step(W, M, [to_device(g, "bf16") for g in grads], v, **HP)
        torch.cuda.synchronize()
        return W, M, v

    Wa, Ma, va = run(G)
    Wb, Mb, vb = run(G_nan)
    for i in (0, 2):
        assert torch.equal(Wb[i], Wa[i]) and torch.equal(Mb[i], Ma[i]) and torch.equal(vb[i], va[i]), i
    ref = oracle.muon_step(stored_f64(W0[1], "bf16"), M0[1].astype(np.float64),
                           stored_f64(G_nan[1], "bf16"), kind="standard",
                           v=v0[1].astype(np.float64), storage="bf16", **HP)
    _nan_aware(to_f64(Mb[1]), ref["M"], 1e-6, "M[1]")
    assert np.isnan(ref["W_exact"]).all() and np.isnan(ref["v"]).all()
    assert torch.isnan(Wb[1].float()).all() and torch.isnan(vb[1]).all()


def test_dion3_nan_row_is_never_selected():
    rows, cols, f = 64, 200, 0.25
    k = oracle.rows_for_fraction(f, rows)
    _say("case Dion3 with a NaN in the top row, 64x200, f = 1/4")
    W0 = synthetic.weight(rows, cols, "bf16", 984, 0)
    M0 = synthetic.state(rows, cols, 985, 0, scale=0.5)
    v0 = np.abs(synthetic.state(rows, 1, 986, 0, scale=0.01)).reshape(rows).astype(np.float32)
    G = synthetic.gradient("student_t", rows, cols, "bf16", 987, 0, 0)
    top = int(oracle.select_rows(M0.astype(np.float64) + stored_f64(G, "bf16"), k)[0])
    G[top, 11] = BF16_NAN
    W = to_device(W0, "bf16")
    M = torch.from_numpy(M0).cuda()
    v = torch.from_numpy(v0).cuda()
    mns.muon_step(W, M, to_device(G, "bf16"), v, kind="gram", restart_before=(3,), row_fraction=f,
                  **HP)
    torch.cuda.synchronize()
    g64, w64 = stored_f64(G, "bf16"), stored_f64(W0, "bf16")
    assert top not in oracle.select_rows(M0.astype(np.float64) + g64, k).tolist()
    ref = oracle.dion3_step(w64, M0.astype(np.float64), g64, f=f, kind="gram", restart_before=(3,),
                            v=v0.astype(np.float64), storage="bf16", **HP)
    assert np.isfinite(to_f64(W)).all()
    check_weight(to_f64(W), w64, ref["W_exact"] - w64, "bf16", "W")
    _nan_aware(to_f64(M), ref["M"], 1e-6, "M")
    assert np.isfinite(to_f64(v)).all() and rel(to_f64(v), ref["v"]) < TOL["bf16"]
