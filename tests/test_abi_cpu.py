"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments synchronously with the documented status codes
(validation happens before any HIP call, so none of these touches a device)."""
import ctypes
import os
import re

import pytest

from muon_newton_schulz_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_ns.h")
QUINTIC = (3.4445, -4.7750, 2.0315)


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


PROBE_HEADER = os.path.join(ROOT, "include", "mns_probe.h")


def _declared_in(header):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_every_header_is_covered():
    # each header under include/ has its library and its list of exports checked here
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["mns_probe.h", "muon_ns.h"]


def test_probe_header_declares_its_exports_and_the_library_exports_them():
    from muon_newton_schulz_amd import probe
    assert sorted(probe.EXPORTS) == _declared_in(PROBE_HEADER)
    lib = probe.load()
    for name in probe.EXPORTS:
        assert hasattr(lib, name), name


def test_probe_rejects_bad_arguments_before_any_hip_call():
    import ctypes
    from muon_newton_schulz_amd import probe
    lib = probe.load()
    f = ctypes.c_double(0.0)
    assert lib.mns_probe_mfma_launch(0, 0, None, ctypes.byref(f)) == 4
    assert lib.mns_probe_mfma_launch(1000001, 0, None, ctypes.byref(f)) == 4
    assert lib.mns_probe_mfma_launch(10, 0, None, None) == 4
    assert lib.mns_probe_mfma_checksum(0, ctypes.byref(f)) == 4
    assert lib.mns_probe_mfma_checksum(10, None) == 4
    # nothing launched yet in this process: no results to read
    assert lib.mns_probe_mfma_checksum(10, ctypes.byref(f)) == 4


def test_header_declares_the_exports():
    assert sorted(_abi.EXPORTS) == _declared_functions()


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.mns_version() == 100
    for code in range(7):
        assert lib.mns_status_string(code).decode().startswith("MNS_")
    assert b"unknown" in lib.mns_status_string(99)


def _hp(T=5, kind=0, mask=0, normuon=0, f=1.0, dtype=_abi.MNS_BF16, beta2=0.95, eps=1e-8,
        coeffs=None):
    vals = list(coeffs) if coeffs is not None else list(QUINTIC) * T
    abc = (ctypes.c_float * max(1, len(vals)))(*vals)
    hp = _abi.MnsHparams(mu=0.95, lr=0.02, T=T, abc=ctypes.cast(abc, ctypes.POINTER(ctypes.c_float)),
                         kind=kind, restart_mask=mask, normuon=normuon, beta2=beta2, eps=eps,
                         row_fraction=f, dtype=dtype)
    return hp, abc


def _mats(shapes, ptr=0x10000):
    arr = (_abi.MnsMatrix * len(shapes))()
    for i, (r, c) in enumerate(shapes):
        arr[i].W = arr[i].M = arr[i].G = arr[i].v = ptr
        arr[i].rows, arr[i].cols = r, c
    return arr


def _ws_size(lib, shapes, **kw):
    hp, keep = _hp(**kw)
    out = ctypes.c_size_t(0)
    st = lib.mns_step_workspace_size(_mats(shapes), len(shapes), ctypes.byref(hp), ctypes.byref(out))
    return st, out.value


def test_workspace_sizes_cover_the_iterates(lib):
    st, b = _ws_size(lib, [(4096, 16384)])
    assert st == 0
    # two float16 iterates of 4096 x 16384 plus two 4096^2 float16 scratch matrices
    assert b >= 2 * 4096 * 16384 * 2 + 2 * 4096 * 4096 * 2
    st, g = _ws_size(lib, [(4096, 16384)], kind=1, mask=1 << 3)
    assert st == 0 and g >= 2 * 4096 * 16384 * 2 + 6 * 4096 * 4096 * 2
    # tall matrices run on the short side: same iterate size as the transpose
    assert _ws_size(lib, [(16384, 4096)])[1] >= 2 * 4096 * 16384 * 2
    # float32 storage doubles the iterate
    assert _ws_size(lib, [(256, 1024)], dtype=_abi.MNS_F32)[1] >= 2 * 256 * 1024 * 4
    # Dion3 with f = 1/4 orthogonalises 1280 of 5120 rows
    st, d = _ws_size(lib, [(5120, 13824)], kind=1, mask=8, normuon=1, f=0.25)
    assert st == 0 and d >= 1280 * 13824 * 4 + 2 * 1280 * 13824 * 2


def test_workspace_is_the_largest_shape_group(lib):
    shapes = [(3072, 3072)] * 4 + [(3072, 8192)] * 2 + [(8192, 3072)]
    st, b = _ws_size(lib, shapes, normuon=1)
    assert st == 0
    assert b == max(_ws_size(lib, [s] * shapes.count(s), normuon=1)[1] for s in set(shapes))


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), _abi.MNS_ERR_PARAM),
    (dict(T=65, coeffs=list(QUINTIC) * 65), _abi.MNS_ERR_PARAM),
    (dict(kind=2), _abi.MNS_ERR_PARAM),
    (dict(kind=0, mask=8), _abi.MNS_ERR_PARAM),          # restarts are Gram-only
    (dict(kind=1, mask=1 << 1), _abi.MNS_ERR_PARAM),     # restart before t = 1 is meaningless
    (dict(kind=1, mask=1 << 6), _abi.MNS_ERR_PARAM),     # beyond T = 5
    (dict(f=0.0), _abi.MNS_ERR_PARAM),
    (dict(f=1.5), _abi.MNS_ERR_PARAM),
    (dict(normuon=1, beta2=1.5), _abi.MNS_ERR_PARAM),
    (dict(normuon=1, eps=-1.0), _abi.MNS_ERR_PARAM),
    (dict(dtype=7), _abi.MNS_ERR_DTYPE),
    (dict(coeffs=[float("nan")] * 15), _abi.MNS_ERR_PARAM),
])
def test_bad_hyperparameters_are_rejected(lib, kw, status):
    assert _ws_size(lib, [(64, 128)], **kw)[0] == status
    hp, keep = _hp(**kw)
    st = lib.muon_step(_mats([(64, 128)]), 1, ctypes.byref(hp), 0x100000, 1 << 30, None)
    assert st == status


@pytest.mark.parametrize("shape", [(0, 10), (10, 0), (65537, 4), (-1, 5), (65536, 65536)])
def test_bad_shapes_are_rejected(lib, shape):
    assert _ws_size(lib, [shape])[0] == _abi.MNS_ERR_SHAPE


def test_iterate_size_rule_counts_the_row_pitch(lib):
    # bf16 iterate rows_p x (cols_p + 256) must stay below 2 GiB: 32768 x (32256 + 256) x 2 B
    # fits, 32768 x (32512 + 256) x 2 B = 2^31 B does not (though rows * cols < 2^31).
    assert _ws_size(lib, [(32768, 32256)])[0] == 0
    assert _ws_size(lib, [(32768, 32512)])[0] == _abi.MNS_ERR_SHAPE
    assert _ws_size(lib, [(32512, 32768)])[0] == _abi.MNS_ERR_SHAPE
    out = ctypes.c_size_t(0)
    assert lib.mns_ns_workspace_size(_abi.MNS_BF16, 1, 32768, 32512, 0, ctypes.byref(out)) == _abi.MNS_ERR_SHAPE


def test_null_and_misaligned_pointers(lib):
    hp, keep = _hp(normuon=1)
    m = _mats([(64, 128)])
    m[0].v = None
    assert lib.muon_step(m, 1, ctypes.byref(hp), 0x100000, 1 << 30, None) == _abi.MNS_ERR_NULL
    m = _mats([(64, 128)], ptr=0x10008)                    # 8-byte aligned only
    assert lib.muon_step(m, 1, ctypes.byref(hp), 0x100000, 1 << 30, None) == _abi.MNS_ERR_PARAM
    assert lib.muon_step(None, 1, ctypes.byref(hp), 0x100000, 1 << 30, None) == _abi.MNS_ERR_NULL
    assert lib.muon_step(_mats([(64, 128)]), 0, ctypes.byref(hp), 0x100000, 1 << 30, None) == _abi.MNS_ERR_SHAPE


def test_workspace_errors(lib):
    hp, keep = _hp()
    m = _mats([(64, 128)])
    st, need = _ws_size(lib, [(64, 128)])
    assert st == 0
    assert lib.muon_step(m, 1, ctypes.byref(hp), None, need, None) == _abi.MNS_ERR_WORKSPACE
    assert lib.muon_step(m, 1, ctypes.byref(hp), 0x100010, need, None) == _abi.MNS_ERR_WORKSPACE
    assert lib.muon_step(m, 1, ctypes.byref(hp), 0x100000, need - 1, None) == _abi.MNS_ERR_WORKSPACE


def test_standalone_entry_points_validate(lib):
    abc = (ctypes.c_float * 15)(*(list(QUINTIC) * 5))
    out = ctypes.c_size_t(0)
    assert lib.mns_ns_workspace_size(_abi.MNS_BF16, 2, 300, 700, 0, ctypes.byref(out)) == 0
    assert out.value >= 2 * 2 * 512 * 768 * 2
    assert lib.mns_ns_workspace_size(5, 1, 8, 8, 0, ctypes.byref(out)) == _abi.MNS_ERR_DTYPE
    assert lib.mns_ns_workspace_size(0, 0, 8, 8, 0, ctypes.byref(out)) == _abi.MNS_ERR_SHAPE
    assert lib.ns_orthogonalize(None, 0x1000, 1, 1, 8, 8, 5, abc, 0x100000, 1 << 20, None) == _abi.MNS_ERR_NULL
    assert lib.ns_orthogonalize(0x1000, 0x1000, 1, 1, 8, 8, 0, abc, 0x100000, 1 << 20, None) == _abi.MNS_ERR_PARAM
    assert lib.ns_orthogonalize(0x1000, 0x2000, 1, 1, 8, 8, 5, None, 0x100000, 1 << 20, None) == _abi.MNS_ERR_NULL
    assert lib.gram_ns_orthogonalize(0x1000, 0x2000, 1, 1, 8, 8, 5, abc, 1 << 7, 0x100000, 1 << 20, None) == _abi.MNS_ERR_PARAM
    assert lib.gram_ns_orthogonalize(0x1000, 0x2000, 1, 1, 8, 8, 5, abc, 8, 0x100000, 16, None) == _abi.MNS_ERR_WORKSPACE
    assert lib.mns_normuon_workspace_size(3, 100, 50, ctypes.byref(out)) == 0 and out.value >= 2 * 300 * 4
    fp = ctypes.POINTER(ctypes.c_float)
    assert lib.normuon_scale(0x1000, 1, 1, 8, 8, ctypes.cast(0x2000, fp), 2.0, 1e-8, 0x100000, 1 << 20, None) == _abi.MNS_ERR_PARAM
    assert lib.normuon_scale(0x1000, 1, 1, 8, 8, None, 0.9, 1e-8, 0x100000, 1 << 20, None) == _abi.MNS_ERR_NULL


def test_noalloc_rejects_oversize_before_any_device_call(lib):
    # 2304 x 4096 bf16 needs more than the 64 MiB device scratch for one matrix: the call
    # must return MNS_ERR_WORKSPACE from the host checks alone (no device is touched here)
    abc = (ctypes.c_float * 15)(*(list(QUINTIC) * 5))
    assert lib.ns_orthogonalize_noalloc(0x1000, 0x200000, _abi.MNS_BF16, 1, 2304, 4096, 5, abc,
                                        None) == _abi.MNS_ERR_WORKSPACE
    assert lib.ns_orthogonalize_noalloc(0x1000, 0x200000, _abi.MNS_BF16, 1, 4096, 2304, 5, abc,
                                        None) == _abi.MNS_ERR_WORKSPACE
    # the usual argument checks come first
    assert lib.ns_orthogonalize_noalloc(None, 0x2000, _abi.MNS_BF16, 1, 8, 8, 5, abc, None) == _abi.MNS_ERR_NULL
    assert lib.ns_orthogonalize_noalloc(0x1000, 0x2000, 7, 1, 8, 8, 5, abc, None) == _abi.MNS_ERR_DTYPE
    assert lib.ns_orthogonalize_noalloc(0x1000, 0x2000, _abi.MNS_BF16, 1, 8, 8, 0, abc, None) == _abi.MNS_ERR_PARAM


def test_profile_session_states(lib):
    """The instrumentation calls outside and inside a session: with nothing launched in it, a
    session makes no device call, so the state rules are checked here."""
    n = ctypes.c_int(-1)
    stats = (_abi.MnsKernelStat * 4)()
    # no session open
    assert lib.mns_profile_set_flush(None, 0) == _abi.MNS_ERR_PARAM
    assert lib.mns_profile_end(stats, 4, ctypes.byref(n)) == _abi.MNS_ERR_PARAM
    assert lib.mns_profile_begin() == _abi.MNS_OK
    try:
        # a flush buffer must be 16-byte aligned; NULL or zero bytes turns the flush off
        assert lib.mns_profile_set_flush(ctypes.c_void_p(0x10008), 1 << 30) == _abi.MNS_ERR_PARAM
        assert lib.mns_profile_set_flush(ctypes.c_void_p(0x10000), 1 << 30) == _abi.MNS_OK
        assert lib.mns_profile_set_flush(None, 0) == _abi.MNS_OK
        assert lib.mns_profile_set_flush(ctypes.c_void_p(0x10000), 0) == _abi.MNS_OK
        # a second begin restarts the session
        assert lib.mns_profile_begin() == _abi.MNS_OK
    finally:
        assert lib.mns_profile_end(stats, 4, ctypes.byref(n)) == _abi.MNS_OK
    assert n.value == 0   # nothing was launched in the session
    # end closes it, and turns the flush off with it
    assert lib.mns_profile_end(stats, 4, ctypes.byref(n)) == _abi.MNS_ERR_PARAM
    assert lib.mns_profile_set_flush(ctypes.c_void_p(0x10000), 1 << 30) == _abi.MNS_ERR_PARAM
