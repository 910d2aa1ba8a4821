"""GPU parity at sizes the oracle finishes in seconds: several 256 x 256 tiles plus ragged
tails, tall and wide, batched, every entry point through the C ABI, against the fp64
oracle. Tolerances: relative Frobenius 2e-2 (bfloat16 storage), 1e-4 (float32)."""
import numpy as np
import pytest
import torch

import oracle
import muon_newton_schulz_amd as mns
import synthetic
from helpers import TOL, check_weight, rel, stored_f64, to_device, to_f64

pytestmark = pytest.mark.gpu
QUINTIC = (3.4445, -4.7750, 2.0315)


def _say(*a):
    print(*a, flush=True)


def _inputs(shape, storage, seed, batch=1, dist="normal"):
    xs = [synthetic.gradient(dist, *shape, storage, 900, seed, i) for i in range(batch)]
    return np.stack(xs)


@pytest.mark.parametrize("storage", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 700), (700, 300), (256, 512), (1, 9), (37, 37)])
@pytest.mark.parametrize("coeff", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (0.5, -0.3, 0.2)])
def test_ns_single_polynomial(storage, shape, coeff):
    """One NS step with one monomial at a time isolates X/||X||, the Gram product X X^T,
    the symmetric product A^2 and the rectangular B X."""
    _say("case", storage, shape, coeff)
    x = _inputs(shape, storage, 1, batch=2)
    X = to_device(x, storage)
    O = mns.ns_orthogonalize(X, [coeff])
    torch.cuda.synchronize()
    got = to_f64(O)
    for b in range(2):
        want = oracle.newton_schulz(stored_f64(x[b], storage), [coeff])
        assert rel(got[b], want) < TOL[storage], (b, rel(got[b], want))


@pytest.mark.parametrize("storage", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 700), (700, 300), (512, 1024), (520, 520)])
def test_ns_quintic(storage, shape):
    _say("case", storage, shape)
    x = _inputs(shape, storage, 2, batch=3, dist="student_t")
    O = mns.ns_orthogonalize(to_device(x, storage), [QUINTIC] * 5)
    torch.cuda.synchronize()
    got = to_f64(O)
    for b in range(3):
        want = oracle.newton_schulz(stored_f64(x[b], storage), [QUINTIC] * 5)
        assert rel(got[b], want) < TOL[storage]


# Work decomposition of the products: 128 x 128 or 256 x 256 output tiles, whole rounds of
# tiles over the CUs, and a last round that is split along k (partial sums added by a second
# launch). The comments give the decomposition on a 256-CU device.
@pytest.mark.parametrize("storage,shape,batch,check", [
    ("bf16", (256, 4096), 2, (0, 1)),          # X X^T: 6 tiles, k split 8 ways
    ("f32", (256, 4096), 2, (0, 1)),           # float32 path: k split 16 ways
    ("bf16", (640, 3000), 1, (0,)),            # ragged padding inside split tiles (6 ways)
    ("bf16", (3000, 640), 1, (0,)),            # the same, tall
    ("bf16", (1024, 2048), 16, (0, 9, 15)),    # 576 tiles: one full round, tail split 4 ways
    ("bf16", (2048, 2048), 15, (0, 14)),       # 256-tiles: two full rounds, tail split 4 ways
])
def test_ns_work_decomposition(storage, shape, batch, check):
    _say("case decomposition", storage, shape, batch)
    x = _inputs(shape, storage, 8, batch=batch, dist="student_t")
    X = to_device(x, storage)
    O = mns.ns_orthogonalize(X, [QUINTIC] * 5)
    G = mns.gram_ns_orthogonalize(X, [QUINTIC] * 5, restart_before=(3,))
    torch.cuda.synchronize()
    got, got_g = to_f64(O), to_f64(G)
    for b in check:
        want = oracle.newton_schulz(stored_f64(x[b], storage), [QUINTIC] * 5)
        assert rel(got[b], want) < TOL[storage], (b, rel(got[b], want))
        want_g = oracle.gram_newton_schulz(stored_f64(x[b], storage), [QUINTIC] * 5, (3,))
        assert rel(got_g[b], want_g) < TOL[storage], (b, rel(got_g[b], want_g))


@pytest.mark.parametrize("storage", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 900), (900, 300), (512, 512)])
@pytest.mark.parametrize("restarts", [(), (3,), (2, 4)])
def test_gram_ns(storage, shape, restarts):
    _say("case", storage, shape, restarts)
    x = _inputs(shape, storage, 3, batch=2)
    O = mns.gram_ns_orthogonalize(to_device(x, storage), [QUINTIC] * 5, restart_before=restarts)
    torch.cuda.synchronize()
    got = to_f64(O)
    for b in range(2):
        want = oracle.gram_newton_schulz(stored_f64(x[b], storage), [QUINTIC] * 5, restarts)
        assert rel(got[b], want) < TOL[storage]


def test_zero_matrix_gives_zero_and_keeps_weights():
    _say("case zero")
    X = torch.zeros(64, 300, dtype=torch.bfloat16, device="cuda")
    assert not mns.ns_orthogonalize(X, [QUINTIC] * 5).any()
    assert not mns.gram_ns_orthogonalize(X, [QUINTIC] * 5).any()
    W = torch.randn(64, 300, device="cuda").to(torch.bfloat16)
    W0 = W.clone()
    M = torch.zeros(64, 300, device="cuda")
    v = torch.zeros(64, device="cuda")
    mns.muon_step(W, M, X, v, mu=0.9, lr=0.1, coeffs=[QUINTIC] * 5, normuon=True)
    torch.cuda.synchronize()
    assert torch.equal(W, W0) and not M.any() and not v.any()


def _step_case(shapes, storage, kind, restarts, normuon, f, seed, steps=1, w_zero=False):
    mu, lr = 0.9, 0.05
    Ws = [synthetic.weight(r, c, storage, 950, i, zero=w_zero) for i, (r, c) in enumerate(shapes)]
    Ms = [synthetic.state(r, c, 950, i, scale=0.5) for i, (r, c) in enumerate(shapes)]
    vs = [np.abs(synthetic.state(r, 1, 951, i, scale=0.01)).reshape(r) for i, (r, c) in enumerate(shapes)]
    W = [to_device(w, storage) for w in Ws]
    M = [torch.from_numpy(m).cuda() for m in Ms]
    v = [torch.from_numpy(x.astype(np.float32)).cuda() for x in vs]
    for step in range(steps):
        Gs = [synthetic.gradient("student_t", r, c, storage, 952, step + seed, i)
              for i, (r, c) in enumerate(shapes)]
        W_before = [to_f64(t) for t in W]
        M_before = [to_f64(t) for t in M]
        v_before = [to_f64(t) for t in v]
        mns.muon_step(W, M, [to_device(g, storage) for g in Gs], v if normuon else None, mu=mu,
                      lr=lr, coeffs=[QUINTIC] * 5, kind=kind, restart_before=restarts,
                      normuon=normuon, beta2=0.9, eps=1e-8, row_fraction=f)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            g64 = stored_f64(Gs[i], storage)
            if f < 1.0:
                ref = oracle.dion3_step(W_before[i], M_before[i], g64, mu=mu, lr=lr, f=f,
                                        coeffs=[QUINTIC] * 5, kind=kind, restart_before=restarts,
                                        normuon=normuon, v=v_before[i], beta2=0.9, eps=1e-8,
                                        storage=storage)
            else:
                ref = oracle.muon_step(W_before[i], M_before[i], g64, mu=mu, lr=lr,
                                       coeffs=[QUINTIC] * 5, kind=kind, restart_before=restarts,
                                       normuon=normuon, v=v_before[i], beta2=0.9, eps=1e-8,
                                       storage=storage)
            check_weight(to_f64(W[i]), W_before[i], ref["W_exact"] - W_before[i], storage,
                         f"W[{i}] step {step}")
            assert rel(to_f64(M[i]), ref["M"]) < 1e-6, f"M[{i}]"
            if normuon:
                assert rel(to_f64(v[i]), ref["v"]) < TOL[storage], f"v[{i}]"


@pytest.mark.parametrize("storage", ["bf16", "f32"])
@pytest.mark.parametrize("normuon", [False, True])
def test_muon_step_mixed_shapes(storage, normuon):
    """Several shapes in one call: grouping by shape, tall and wide, ragged sizes."""
    _say("case", storage, normuon)
    shapes = [(300, 700), (300, 700), (700, 300), (256, 256), (300, 700)]
    _step_case(shapes, storage, "standard", (), normuon, 1.0, 0, steps=2)


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_muon_step_gram_kind(storage):
    _say("case", storage)
    _step_case([(260, 1100), (1100, 260)], storage, "gram", (3,), True, 1.0, 10)


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_normuon_row_sums_from_split_tail(storage):
    """NorMuon's row statistics come from the epilogue of the product that writes the NS
    result. At 1024 x 1536 that product's last round of tiles is split along k, so they come
    from the split-tail epilogue: C's rows for the wide matrix, C^T's for the tall one."""
    _say("case normuon split tail", storage)
    _step_case([(1024, 1536), (1536, 1024)], storage, "standard", (), True, 1.0, 40)


def test_muon_step_many_matrices_one_shape():
    """More matrices of one shape than one batched launch holds (32: chunking)."""
    _say("case 40 x 128x384")
    _step_case([(128, 384)] * 40, "bf16", "standard", (), True, 1.0, 20, w_zero=True)


@pytest.mark.parametrize("shape,f", [((64, 200), 0.25), ((200, 64), 0.5), ((100, 300), 1.0 / 3)])
def test_dion3_step(shape, f):
    _say("case dion3", shape, f)
    _step_case([shape, shape], "bf16", "gram", (3,), True, f, 30, steps=3)


def test_dion3_selection_matches_oracle():
    """Top-k rows by l1 with ties to the lower index: exact indices (the ties here are exact
    in float32: duplicated rows)."""
    _say("case dion3 ties")
    rows, cols = 44, 96
    rng = np.random.default_rng(5)
    base = rng.standard_normal((rows // 2, cols)).astype(np.float32)
    G = np.concatenate([base, base[::-1]], axis=0)           # every l1 norm appears twice
    # k = ceil(44 / 4) = 11 splits one tied pair: its lower-index row must win
    W = torch.zeros(rows, cols, device="cuda")
    M = torch.zeros(rows, cols, device="cuda")
    mns.muon_step(W, M, torch.from_numpy(G).cuda(), mu=0.5, lr=0.1, coeffs=[QUINTIC] * 5,
                  kind="gram", restart_before=(3,), row_fraction=0.25)
    torch.cuda.synchronize()
    S = oracle.select_rows(G.astype(np.float64), 11)
    decayed = np.where(np.isclose(M.cpu().numpy(), 0.5 * G).all(axis=1) & ~np.isclose(G, 0).all(axis=1))[0]
    assert sorted(decayed.tolist()) == sorted(S.tolist())
    moved = np.where(W.cpu().numpy().any(axis=1))[0]
    assert sorted(moved.tolist()) == sorted(S.tolist())


def test_dion3_selection_all_ties():
    """Every row has the same l1 norm (identical rows): each radix pass ties on every key,
    and the k rows of lowest index are taken (k = ceil(300 / 4) = 75)."""
    _say("case dion3 all ties")
    rows, cols = 300, 64
    rng = np.random.default_rng(8)
    G = np.tile(rng.standard_normal((1, cols)).astype(np.float32), (rows, 1))
    W = torch.zeros(rows, cols, device="cuda")
    M = torch.zeros(rows, cols, device="cuda")
    mns.muon_step(W, M, torch.from_numpy(G).cuda(), mu=0.5, lr=0.1, coeffs=[QUINTIC] * 5,
                  kind="gram", restart_before=(3,), row_fraction=0.25)
    torch.cuda.synchronize()
    want = oracle.select_rows(G.astype(np.float64), 75)
    assert sorted(want.tolist()) == list(range(75))
    moved = np.where(W.cpu().numpy().any(axis=1))[0]
    assert moved.tolist() == list(range(75))
    decayed = np.where(np.isclose(M.cpu().numpy(), 0.5 * G).all(axis=1))[0]
    assert decayed.tolist() == list(range(75))


@pytest.mark.parametrize("rows,pattern", [(9001, "all_ties"), (12004, "pairs")])
def test_dion3_selection_many_rows(rows, pattern):
    """More rows than the selection keeps in registers (over 8 per thread of its 1024), so it
    reads the norms in chunks: the tie order must still follow the row index across the
    chunks and the threads. "pairs": every l1 norm appears twice, far apart, and k is odd, so
    one tied pair is split; "all_ties": identical rows, the k of lowest index win."""
    _say("case dion3 many rows", rows, pattern)
    cols = 64
    rng = np.random.default_rng(rows)
    if pattern == "pairs":
        # scaled copies of one row, scales 1/rows apart (far above float32's rounding of an
        # l1 sum), so the float32 and float64 orders agree; each row appears twice
        v = rng.standard_normal(cols).astype(np.float32)
        scale = (1.0 + rng.permutation(rows // 2) / rows).astype(np.float32)
        base = scale[:, None] * v[None, :]
        G = np.concatenate([base, base[::-1]], axis=0)
    else:
        G = np.tile(rng.standard_normal((1, cols)).astype(np.float32), (rows, 1))
    k = oracle.rows_for_fraction(0.25, rows)
    assert k % 2 == 1
    W = torch.zeros(rows, cols, device="cuda")
    M = torch.zeros(rows, cols, device="cuda")
    mns.muon_step(W, M, torch.from_numpy(G).cuda(), mu=0.5, lr=0.1, coeffs=[QUINTIC] * 5,
                  kind="gram", restart_before=(3,), row_fraction=0.25)
    torch.cuda.synchronize()
    want = np.sort(oracle.select_rows(G.astype(np.float64), k))
    if pattern == "all_ties":
        assert want.tolist() == list(range(k))
    moved = np.where(W.cpu().numpy().any(axis=1))[0]
    assert moved.tolist() == want.tolist()
    decayed = np.where(np.isclose(M.cpu().numpy(), 0.5 * G).all(axis=1))[0]
    assert decayed.tolist() == want.tolist()


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_normuon_scale(storage):
    _say("case normuon", storage)
    rng = np.random.default_rng(6)
    o = (rng.standard_normal((3, 70, 130)) * rng.uniform(0.2, 2.0, (3, 70, 1))).astype(np.float32)
    stored = synthetic.encode(o, storage)
    v0 = rng.uniform(0, 0.1, (3, 70)).astype(np.float32)
    O = to_device(stored, storage)
    v = torch.from_numpy(v0.copy()).cuda()
    mns.normuon_scale(O, v, beta2=0.9, eps=1e-6)
    torch.cuda.synchronize()
    got, gv = to_f64(O), to_f64(v)
    for b in range(3):
        vn, u = oracle.normuon_update(stored_f64(stored[b], storage), v0[b].astype(np.float64), 0.9, 1e-6)
        assert rel(got[b], u) < TOL[storage] * 0.5
        assert rel(gv[b], vn) < 1e-5


def test_repeat_runs_are_bitwise_identical():
    _say("case determinism")
    x = _inputs((520, 1400), "bf16", 7, batch=2)
    X = to_device(x, "bf16")
    a = mns.ns_orthogonalize(X, [QUINTIC] * 5)
    b = mns.ns_orthogonalize(X, [QUINTIC] * 5)
    c = mns.gram_ns_orthogonalize(X, [QUINTIC] * 5)
    d = mns.gram_ns_orthogonalize(X, [QUINTIC] * 5)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


@pytest.mark.parametrize("kind,f", [("standard", 1.0), ("gram", 1.0), ("standard", 0.25)])
def test_zero_matrices_among_others(kind, f):
    """Matrices whose momentum and gradient are zero, batched with non-zero ones of the same
    shape: each matrix has its own scale in the one launch sequence, so the zero ones keep W
    bit for bit and M at zero, with v decayed by beta2 (their NorMuon ratio is 0/0, taken as
    0), and the others still match the oracle (standard NS, Gram NS, Dion3 rows)."""
    _say("case zero among others", kind, f)
    shapes = [(300, 700)] * 4
    zero = {1, 3}
    mu, lr, beta2 = 0.9, 0.05, 0.9
    Ws = [synthetic.weight(r, c, "bf16", 960, i) for i, (r, c) in enumerate(shapes)]
    Ms = [np.zeros((r, c)) if i in zero else synthetic.state(r, c, 960, i, scale=0.5)
          for i, (r, c) in enumerate(shapes)]
    # bfloat16 storage: the gradients are bit patterns (0x0000 is +0.0)
    Gs = [np.zeros((r, c), dtype=np.uint16) if i in zero
          else synthetic.gradient("student_t", r, c, "bf16", 961, 0, i)
          for i, (r, c) in enumerate(shapes)]
    vs = [np.abs(synthetic.state(r, 1, 962, i, scale=0.01)).reshape(r) for i, (r, c) in enumerate(shapes)]
    W = [to_device(w, "bf16") for w in Ws]
    M = [torch.from_numpy(m).float().cuda() for m in Ms]
    v = [torch.from_numpy(x.astype(np.float32)).cuda() for x in vs]
    W_before = [to_f64(t) for t in W]
    W_bits = [t.clone() for t in W]
    v_before = [to_f64(t) for t in v]
    mns.muon_step(W, M, [to_device(g, "bf16") for g in Gs], v, mu=mu, lr=lr,
                  coeffs=[QUINTIC] * 5, kind=kind, restart_before=(3,) if kind == "gram" else (),
                  normuon=True, beta2=beta2, eps=1e-8, row_fraction=f)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.isfinite(W[i].float()).all() and torch.isfinite(v[i]).all(), f"non-finite [{i}]"
        if i in zero:
            assert torch.equal(W[i], W_bits[i]), f"W[{i}] changed"
            assert not M[i].any(), f"M[{i}] not zero"
            # rows of the zero matrix: v <- beta2 v (every row, or the selected rows for Dion3)
            vv = to_f64(v[i])
            decayed = np.isclose(vv, beta2 * v_before[i], rtol=1e-6, atol=0)
            kept = np.isclose(vv, v_before[i], rtol=0, atol=0)
            assert decayed.all() if f == 1.0 else (decayed | kept).all(), f"v[{i}]"
            continue
        g64 = stored_f64(Gs[i], "bf16")
        kw = dict(coeffs=[QUINTIC] * 5, kind=kind, restart_before=(3,) if kind == "gram" else (),
                  normuon=True, v=v_before[i], beta2=beta2, eps=1e-8, storage="bf16")
        if f < 1.0:
            ref = oracle.dion3_step(W_before[i], np.asarray(Ms[i], dtype=np.float64), g64, mu=mu,
                                    lr=lr, f=f, **kw)
        else:
            ref = oracle.muon_step(W_before[i], np.asarray(Ms[i], dtype=np.float64), g64, mu=mu,
                                   lr=lr, **kw)
        check_weight(to_f64(W[i]), W_before[i], ref["W_exact"] - W_before[i], "bf16", f"W[{i}]")
        assert rel(to_f64(M[i]), ref["M"]) < 1e-6, f"M[{i}]"
        assert rel(to_f64(v[i]), ref["v"]) < TOL["bf16"], f"v[{i}]"


@pytest.mark.parametrize("storage", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [1e-24, 1e24])
def test_extreme_scales(storage, scale):
    """The orthogonalisation is scale-free (X_0 = M / ||M||_F): momenta and gradients whose
    squares underflow (1e-24) or overflow (1e24) float32 give the same step as the oracle's,
    through the step (k_momentum's norm) and the standalone entry point (k_sumsq's)."""
    _say("case extreme scale", storage, scale)
    r, c, mu, lr = 300, 700, 0.9, 0.05
    W = to_device(synthetic.weight(r, c, storage, 970, 0), storage)
    M0 = synthetic.state(r, c, 970, 0, scale=0.5).astype(np.float64) * scale
    g = synthetic.gradient("student_t", r, c, "f32", 971, 0, 0).astype(np.float64) * scale
    G = (torch.from_numpy(g.astype(np.float32)).cuda() if storage == "f32"
         else torch.from_numpy(g.astype(np.float32)).cuda().to(torch.bfloat16))
    M = torch.from_numpy(M0.astype(np.float32)).cuda()
    W_before, M_before, g64 = to_f64(W), to_f64(M), to_f64(G)
    mns.muon_step([W], [M], [G], None, mu=mu, lr=lr, coeffs=[QUINTIC] * 5)
    torch.cuda.synchronize()
    ref = oracle.muon_step(W_before, M_before, g64, mu=mu, lr=lr, coeffs=[QUINTIC] * 5,
                           storage=storage)
    check_weight(to_f64(W), W_before, ref["W_exact"] - W_before, storage, "W")
    assert rel(to_f64(M), ref["M"]) < 1e-6
    # the standalone orthogonalisation of the gradient itself
    O = mns.ns_orthogonalize(G, [QUINTIC] * 5)
    torch.cuda.synchronize()
    O_ref = oracle.newton_schulz(g64, [QUINTIC] * 5)
    assert torch.isfinite(O.float()).all()
    assert rel(to_f64(O), O_ref) < TOL[storage]
