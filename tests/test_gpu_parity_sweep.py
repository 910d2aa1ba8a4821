"""A seeded sweep of ragged shapes and batch sizes through both Newton-Schulz entry points,
through one grouped step and through Dion3 steps at several row fractions, against the fp64
oracle: sizes on either side of the 64-, 128- and 256-element tile and padding boundaries,
below one tile and just past one, wide and tall, single and batched. The cases come from a
fixed generator (the same on every run). Tolerances as elsewhere: relative Frobenius 2e-2
(bfloat16 storage), 1e-4 (float32)."""
import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as mns
import oracle
import synthetic
from helpers import TOL, check_weight, rel, stored_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)
EDGES = [1, 3, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 383, 384, 385, 511, 512, 513, 640]


def _cases(n=20, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        r, c = (int(x) for x in rng.choice(EDGES, size=2))
        out.append((f"{i:02d}", r, c, int(rng.integers(1, 4)), ("standard", "gram")[i % 2],
                    ("bf16", "f32")[(i // 2) % 2]))
    return out


CASES = _cases()


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_{c[1]}x{c[2]}_b{c[3]}_{c[4]}_{c[5]}" for c in CASES])
def test_orthogonalize_sweep(case):
    idx, r, c, batch, kind, storage = case
    _say("case", idx, (r, c), batch, kind, storage)
    x = np.stack([synthetic.gradient("student_t", r, c, storage, 990, int(idx), i) for i in range(batch)])
    X = to_device(x, storage)
    coeffs = [QUINTIC] * 5
    if kind == "standard":
        O = mns.ns_orthogonalize(X, coeffs)
    else:
        O = mns.gram_ns_orthogonalize(X, coeffs, restart_before=(3,))
    torch.cuda.synchronize()
    got = to_f64(O)
    for b in range(batch):
        x64 = stored_f64(x[b], storage)
        want = (oracle.newton_schulz(x64, coeffs) if kind == "standard"
                else oracle.gram_newton_schulz(x64, coeffs, restart_before=(3,)))
        assert rel(got[b], want) < TOL[storage], (b, rel(got[b], want))


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_grouped_step_sweep(storage):
    """One NorMuon step over eight matrices of the sweep's shapes (three share a shape, so one
    group is batched), each against the oracle's step from the same state."""
    shapes = [(c[1], c[2]) for c in CASES[:5]] + [(300, 513)] * 3
    _say("grouped step", storage, shapes)
    mu, lr = 0.9, 0.05
    W0 = [synthetic.weight(r, c, storage, 991, i) for i, (r, c) in enumerate(shapes)]
    M0 = [synthetic.state(r, c, 992, i, scale=0.5) for i, (r, c) in enumerate(shapes)]
    v0 = [np.abs(synthetic.state(r, 1, 993, i, scale=0.01)).reshape(r).astype(np.float32)
          for i, (r, c) in enumerate(shapes)]
    G = [synthetic.gradient("student_t", r, c, storage, 994, 0, i) for i, (r, c) in enumerate(shapes)]
    W = [to_device(w, storage) for w in W0]
    M = [torch.from_numpy(m).cuda() for m in M0]
    v = [torch.from_numpy(x).cuda() for x in v0]
    mns.muon_step(W, M, [to_device(g, storage) for g in G], v, mu=mu, lr=lr, coeffs=[QUINTIC] * 5,
                  normuon=True, beta2=0.9, eps=1e-8)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        w64 = stored_f64(W0[i], storage)
        ref = oracle.muon_step(w64, M0[i].astype(np.float64), stored_f64(G[i], storage), mu=mu, lr=lr,
                               coeffs=[QUINTIC] * 5, normuon=True, v=v0[i].astype(np.float64),
                               beta2=0.9, eps=1e-8, storage=storage)
        check_weight(to_f64(W[i]), w64, ref["W_exact"] - w64, storage, f"W[{i}] {shapes[i]}")
        assert rel(to_f64(M[i]), ref["M"]) < 1e-6, f"M[{i}]"
        assert rel(to_f64(v[i]), ref["v"]) < TOL[storage], f"v[{i}]"


def _dion3_cases(n=6, seed=2027):
    rng = np.random.default_rng(seed)
    fracs = [0.125, 0.25, 1.0 / 3, 0.5, 0.9]
    out = []
    for i in range(n):
        r, c = (int(x) for x in rng.choice(EDGES[2:], size=2))   # at least 63 rows
        out.append((f"{i:02d}", r, c, float(rng.choice(fracs)), ("gram", "standard")[i % 2]))
    return out


DION3_CASES = _dion3_cases()


@pytest.mark.parametrize("case", DION3_CASES,
                         ids=[f"{c[0]}_{c[1]}x{c[2]}_f{c[3]:.3f}_{c[4]}" for c in DION3_CASES])
def test_dion3_sweep(case):
    """Dion3 steps (NorMuon on the selected rows) over the sweep's shapes and several row
    fractions, with Gram and with standard NS, against the oracle's step from the same state
    (the oracle's own selection: random data leaves no near ties at the k-th row)."""
    idx, r, c, f, kind = case
    _say("dion3", idx, (r, c), f, kind)
    mu, lr = 0.9, 0.05
    restarts = (3,) if kind == "gram" else ()
    W0 = synthetic.weight(r, c, "bf16", 995, int(idx))
    M0 = synthetic.state(r, c, 996, int(idx), scale=0.5)
    v0 = np.abs(synthetic.state(r, 1, 997, int(idx), scale=0.01)).reshape(r).astype(np.float32)
    G = synthetic.gradient("student_t", r, c, "bf16", 998, 0, int(idx))
    W = to_device(W0, "bf16")
    M = torch.from_numpy(M0).cuda()
    v = torch.from_numpy(v0).cuda()
    mns.muon_step(W, M, to_device(G, "bf16"), v, mu=mu, lr=lr, coeffs=[QUINTIC] * 5, kind=kind,
                  restart_before=restarts, normuon=True, beta2=0.9, eps=1e-8, row_fraction=f)
    torch.cuda.synchronize()
    w64 = stored_f64(W0, "bf16")
    ref = oracle.dion3_step(w64, M0.astype(np.float64), stored_f64(G, "bf16"), mu=mu, lr=lr, f=f,
                            coeffs=[QUINTIC] * 5, kind=kind, restart_before=restarts, normuon=True,
                            v=v0.astype(np.float64), beta2=0.9, eps=1e-8, storage="bf16")
    check_weight(to_f64(W), w64, ref["W_exact"] - w64, "bf16", "W")
    assert rel(to_f64(M), ref["M"]) < 1e-6, "M"
    assert rel(to_f64(v), ref["v"]) < TOL["bf16"], "v"
