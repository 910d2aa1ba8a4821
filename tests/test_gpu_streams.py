"""Calls on two streams at once, each with its own workspace: the library keeps no state between
calls and is reentrant, so every result must equal, bit for bit, the same call run alone (every
kernel of the path is deterministic)."""
import numpy as np
import pytest
import torch

import muon_newton_schulz_amd as mns
import synthetic
from helpers import to_device

pytestmark = pytest.mark.gpu

QUINTIC = (3.4445, -4.7750, 2.0315)


def _say(*a):
    print(*a, flush=True)


def _batch(shape, batch, seed):
    r, c = shape
    return torch.stack([to_device(synthetic.gradient("student_t", r, c, "bf16", seed, 0, i), "bf16")
                        for i in range(batch)])


def test_orthogonalize_on_two_streams_equals_alone():
    _say("standard NS 3 x 512x1536 on one stream, Gram NS 2 x 768x768 on another")
    coeffs = [QUINTIC] * 5
    X1, X2 = _batch((512, 1536), 3, 970), _batch((768, 768), 2, 971)
    ws1 = torch.empty(mns.ns_workspace_size(X1, "standard"), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(mns.ns_workspace_size(X2, "gram"), dtype=torch.uint8, device="cuda")
    O1, O2 = torch.empty_like(X1), torch.empty_like(X2)
    # alone, one after the other
    mns.ns_orthogonalize(X1, coeffs, out=O1, workspace=ws1)
    torch.cuda.synchronize()
    ref1 = O1.clone()
    mns.gram_ns_orthogonalize(X2, coeffs, restart_before=(3,), out=O2, workspace=ws2)
    torch.cuda.synchronize()
    ref2 = O2.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        O1.zero_()
        O2.zero_()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        for _ in range(2):   # several calls in flight on each stream
            with torch.cuda.stream(s1):
                mns.ns_orthogonalize(X1, coeffs, out=O1, workspace=ws1, stream=s1)
            with torch.cuda.stream(s2):
                mns.gram_ns_orthogonalize(X2, coeffs, restart_before=(3,), out=O2, workspace=ws2,
                                          stream=s2)
        torch.cuda.current_stream().wait_stream(s1)
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        assert torch.equal(O1, ref1), rep
        assert torch.equal(O2, ref2), rep


def test_muon_step_on_two_streams_equals_alone():
    _say("NorMuon step on {300x700, 700x300} and Dion3 step on {256x1024} on two streams")
    common = dict(mu=0.9, lr=0.05, coeffs=[QUINTIC] * 5, beta2=0.9, eps=1e-8)
    sets = [
        ([(300, 700), (700, 300)], dict(kind="standard", normuon=True, row_fraction=1.0)),
        ([(256, 1024)], dict(kind="gram", restart_before=(3,), normuon=True, row_fraction=0.25)),
    ]

    def state(k, shapes):
        W = [to_device(synthetic.weight(r, c, "bf16", 972 + k, i), "bf16") for i, (r, c) in enumerate(shapes)]
        M = [torch.from_numpy(synthetic.state(r, c, 974 + k, i, scale=0.5)).cuda()
             for i, (r, c) in enumerate(shapes)]
        V = [torch.from_numpy(np.abs(synthetic.state(r, 1, 976 + k, i, scale=0.01)).reshape(r)
                              .astype(np.float32)).cuda() for i, (r, c) in enumerate(shapes)]
        G = [to_device(synthetic.gradient("student_t", r, c, "bf16", 978 + k, 0, i), "bf16")
             for i, (r, c) in enumerate(shapes)]
        return W, M, V, G

    init = [state(k, shapes) for k, (shapes, _) in enumerate(sets)]
    wss = [torch.empty(mns.step_workspace_size(W, M, G, V, **common, **kw), dtype=torch.uint8,
                       device="cuda") for (W, M, V, G), (_, kw) in zip(init, sets)]
    # alone
    refs = []
    for (W, M, V, G), (_, kw), ws in zip(init, sets, wss):
        Wc, Mc, Vc = [t.clone() for t in W], [t.clone() for t in M], [t.clone() for t in V]
        mns.muon_step(Wc, Mc, G, Vc, workspace=ws, **common, **kw)
        torch.cuda.synchronize()
        refs.append((Wc, Mc, Vc))
    # together
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = [tuple([t.clone() for t in part] for part in (W, M, V)) for (W, M, V, _G) in init]
    torch.cuda.synchronize()
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for (Wc, Mc, Vc), (_W, _M, _V, G), (_, kw), ws, s in zip(runs, init, sets, wss, streams):
        with torch.cuda.stream(s):
            mns.muon_step(Wc, Mc, G, Vc, workspace=ws, stream=s, **common, **kw)
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k, ((Wc, Mc, Vc), (Wr, Mr, Vr)) in enumerate(zip(runs, refs)):
        for i in range(len(Wc)):
            assert torch.equal(Wc[i], Wr[i]), (k, i, "W")
            assert torch.equal(Mc[i], Mr[i]), (k, i, "M")
            assert torch.equal(Vc[i], Vr[i]), (k, i, "v")
