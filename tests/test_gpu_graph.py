"""The Muon step under HIP graph capture (the grouped step recorded once and replayed, to
remove per-launch overhead on small matrices): every replay, with the program's own eager
work and synchronisations between replays, must equal the same step run eagerly, bit for
bit (every kernel of the step is deterministic), and must match the fp64 oracle's step
from the same pre-step state (W, M, v) to the parity gate."""
import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as mns
import oracle
import synthetic
from helpers import TOL, check_weight, dion3_rows_used, rel, stored_f64, to_device, to_f64

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)


def _say(*a):
    print(*a, flush=True)


CASES = {
    "grouped_standard_normuon": ([(300, 700), (300, 700), (700, 300), (256, 512)],
                                 dict(kind="standard", normuon=True, row_fraction=1.0)),
    "dion3_gram_normuon": ([(512, 1400), (512, 1400)],
                           dict(kind="gram", restart_before=(3,), normuon=True, row_fraction=0.25)),
    "plain_muon_f32": ([(256, 1024)], dict(kind="standard", normuon=False, row_fraction=1.0)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_step_graph_replays_match_eager(case):
    shapes, kw = CASES[case]
    storage = "f32" if case.endswith("f32") else "bf16"
    _say("case", case)
    common = dict(mu=0.9, lr=0.05, coeffs=[QUINTIC] * 5, beta2=0.9, eps=1e-8, **kw)
    W0 = [to_device(synthetic.weight(r, c, storage, 960, i), storage) for i, (r, c) in enumerate(shapes)]
    M0 = [torch.from_numpy(synthetic.state(r, c, 961, i, scale=0.5)).cuda() for i, (r, c) in enumerate(shapes)]
    V0 = [torch.from_numpy(np.abs(synthetic.state(r, 1, 962, i, scale=0.01)).reshape(r).astype(np.float32)).cuda()
          for i, (r, c) in enumerate(shapes)]
    Wg, Mg, Vg = [t.clone() for t in W0], [t.clone() for t in M0], [t.clone() for t in V0]
    We, Me, Ve = [t.clone() for t in W0], [t.clone() for t in M0], [t.clone() for t in V0]
    Ws, Ms, Vs = [t.clone() for t in W0], [t.clone() for t in M0], [t.clone() for t in V0]
    G = [torch.empty_like(w) for w in W0]                       # static gradient buffers
    need = mns.step_workspace_size(Wg, Mg, G, Vg, **common)
    ws_g = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_e = torch.empty(need, dtype=torch.uint8, device="cuda")

    def fill_gradients(step):
        for i, (r, c) in enumerate(shapes):
            G[i].copy_(to_device(synthetic.gradient("student_t", r, c, storage, 963, step, i), storage))

    # warm-up call on scratch state, then capture one step on the capture stream
    fill_gradients(99)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mns.muon_step(Ws, Ms, G, Vs, workspace=ws_g, stream=side, **common)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mns.muon_step(Wg, Mg, G, Vg, workspace=ws_g, stream=torch.cuda.current_stream(), **common)
    torch.cuda.synchronize()
    okw = dict(mu=common["mu"], lr=common["lr"], coeffs=common["coeffs"], kind=common["kind"],
               restart_before=common.get("restart_before", ()), normuon=common["normuon"],
               beta2=common["beta2"], eps=common["eps"], storage=storage)
    f = common["row_fraction"]
    for step in range(4):
        fill_gradients(step)                      # eager work between replays
        torch.cuda.synchronize()
        pre = [(to_f64(Wg[i]), to_f64(Mg[i]), to_f64(Vg[i])) for i in range(len(shapes))]
        graph.replay()
        torch.cuda.synchronize()
        mns.muon_step(We, Me, G, Ve, workspace=ws_e, **common)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(Wg[i], We[i]), (step, i, "W")
            assert torch.equal(Mg[i], Me[i]), (step, i, "M")
            assert torch.equal(Vg[i], Ve[i]), (step, i, "v")
        assert any(not torch.equal(Wg[i], W0[i]) for i in range(len(shapes)))
        # the replayed step against the oracle's step from the same pre-step state
        errs = []
        for i, (r, c) in enumerate(shapes):
            W_pre, M_pre, V_pre = pre[i]
            g64 = stored_f64(synthetic.gradient("student_t", r, c, storage, 963, step, i), storage)
            W1, M1, V1 = to_f64(Wg[i]), to_f64(Mg[i]), to_f64(Vg[i])
            v_in = V_pre if common["normuon"] else None
            if f < 1.0:
                k = oracle.rows_for_fraction(f, r)
                rows = dion3_rows_used(M_pre, g64, M1, W_pre, W1, k, f"replay {step} matrix {i}")
                ref = oracle.dion3_step(W_pre, M_pre, g64, f=f, rows=rows, v=v_in, **okw)
            else:
                ref = oracle.muon_step(W_pre, M_pre, g64, v=v_in, **okw)
            assert rel(M1, ref["M"]) < 1e-6, (step, i, "M")
            if common["normuon"]:
                assert rel(V1, ref["v"]) < TOL[storage], (step, i, "v")
            errs.append(check_weight(W1, W_pre, ref["W_exact"] - W_pre, storage,
                                     f"replay {step} W[{i}]"))
        _say(f"  replay {step}: identical to the eager step; vs oracle worst update rel err "
             f"{max(errs):.2e}")
