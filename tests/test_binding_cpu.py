"""Argument checks of the Python binding that need no GPU: every mismatch the kernels would
turn into an out-of-bounds access or a host pointer on the device must raise before the
library is called. Structural checks (shape, dtype, contiguity, overlap) run first, so CPU
tensors exercise them; otherwise valid CPU tensors must fail the device check."""
import pytest
import torch

import muon_newton_schulz_amd as mns

QUINTIC = (3.4445, -4.7750, 2.0315)
C5 = [QUINTIC] * 5


def _step(W, M, G, v=None, **kw):
    args = dict(mu=0.9, lr=0.02, coeffs=C5)
    args.update(kw)
    mns.muon_step(W, M, G, v, **args)


def _mats(r=64, c=128, dt=torch.bfloat16):
    return (torch.zeros(r, c, dtype=dt), torch.zeros(r, c), torch.zeros(r, c, dtype=dt),
            torch.zeros(r))


def test_cpu_tensors_are_refused():
    W, M, G, v = _mats()
    with pytest.raises(ValueError, match="GPU"):
        _step(W, M, G, v, normuon=True)
    with pytest.raises(ValueError, match="GPU"):
        mns.ns_orthogonalize(G, C5)
    with pytest.raises(ValueError, match="GPU"):
        mns.gram_ns_orthogonalize(G, C5)
    with pytest.raises(ValueError, match="GPU"):
        mns.normuon_scale(G, v)


def test_mixed_storage_dtypes_are_refused():
    W, M, G, v = _mats()
    W2, M2, G2, v2 = _mats(dt=torch.float32)
    with pytest.raises(TypeError, match="storage dtype"):
        _step([W, W2], [M, M2], [G, G2])
    with pytest.raises(TypeError, match="storage dtype"):
        _step([W], [M], [G.float()])                  # G float32 beside a bf16 W
    with pytest.raises(TypeError, match="storage dtype"):
        _step([W, W], [M, M], [G, G2])                # second G float32


def test_unsupported_dtype_is_refused():
    W, M, G, v = _mats(dt=torch.float16)
    with pytest.raises(TypeError):
        _step(W, M, G)
    with pytest.raises(TypeError):
        mns.ns_orthogonalize(G, C5)


def test_momentum_must_be_float32():
    W, M, G, v = _mats()
    with pytest.raises(TypeError, match="momentum"):
        _step(W, M.double(), G)


def test_v_must_be_float32_rows():
    W, M, G, v = _mats()
    with pytest.raises(ValueError, match="v must be float32"):
        _step(W, M, G, v.double(), normuon=True)
    with pytest.raises(ValueError, match="v must be float32"):
        _step(W, M, G, torch.zeros(W.shape[0] + 1), normuon=True)
    with pytest.raises(ValueError, match="v must be float32"):
        _step(W, M, G, torch.zeros(W.shape[0], 1), normuon=True)
    with pytest.raises(ValueError, match="NorMuon needs v"):
        _step(W, M, G, None, normuon=True)
    with pytest.raises(ValueError, match="v must be float32"):
        mns.normuon_scale(G, torch.zeros(G.shape[0], dtype=torch.float64))


def test_shapes_and_counts_must_match():
    W, M, G, v = _mats()
    with pytest.raises(ValueError, match="same shape"):
        _step(W, M[:, :64].contiguous(), G)
    with pytest.raises(ValueError, match="same number"):
        _step([W, W], [M], [G, G])
    with pytest.raises(ValueError, match="contiguous"):
        _step(W.t(), M.t(), G.t())


def test_out_must_match_x():
    W, M, G, v = _mats()
    with pytest.raises(ValueError, match="shape and dtype"):
        mns.ns_orthogonalize(G, C5, out=torch.empty(64, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape and dtype"):
        mns.gram_ns_orthogonalize(G, C5, out=torch.empty(64, 128))
    with pytest.raises(ValueError, match="overlap"):
        mns.ns_orthogonalize(G, C5, out=G)


def test_restart_indices_are_checked():
    assert mns.restart_mask((3,)) == 8
    assert mns.restart_mask((2, 31)) == (1 << 2) | (1 << 31)
    for bad in ((1,), (0,), (32,), (40,)):
        with pytest.raises(ValueError, match="restart"):
            mns.restart_mask(bad)
    with pytest.raises(ValueError, match="restart"):
        mns.restart_mask((6,), T=5)
    W, M, G, v = _mats()
    with pytest.raises(ValueError, match="restart"):
        _step(W, M, G, kind="gram", restart_before=(33,), coeffs=[QUINTIC] * 40)
    with pytest.raises(ValueError, match="kind"):
        _step(W, M, G, kind="cubic")
