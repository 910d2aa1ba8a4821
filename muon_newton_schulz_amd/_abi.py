"""ctypes declarations mirroring include/muon_ns.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon_ns.so")

MNS_OK = 0
MNS_ERR_NULL = 1
MNS_ERR_SHAPE = 2
MNS_ERR_DTYPE = 3
MNS_ERR_PARAM = 4
MNS_ERR_WORKSPACE = 5
MNS_ERR_HIP = 6

MNS_F32 = 0
MNS_BF16 = 1

MNS_NS_STANDARD = 0
MNS_NS_GRAM = 1

# Every symbol include/muon_ns.h declares.
EXPORTS = (
    "mns_status_string", "mns_version", "mns_step_workspace_size", "muon_step",
    "mns_ns_workspace_size", "ns_orthogonalize", "gram_ns_orthogonalize",
    "mns_normuon_workspace_size", "normuon_scale", "mns_profile_begin", "mns_profile_end",
    "mns_profile_set_flush", "ns_orthogonalize_noalloc",
)


class MnsMatrix(ctypes.Structure):
    _fields_ = [
        ("W", ctypes.c_void_p),
        ("M", ctypes.c_void_p),
        ("G", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
    ]


class MnsHparams(ctypes.Structure):
    _fields_ = [
        ("mu", ctypes.c_float),
        ("lr", ctypes.c_float),
        ("T", ctypes.c_int32),
        ("abc", ctypes.POINTER(ctypes.c_float)),
        ("kind", ctypes.c_int32),
        ("restart_mask", ctypes.c_uint32),
        ("normuon", ctypes.c_int32),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("row_fraction", ctypes.c_double),
        ("dtype", ctypes.c_int32),
    ]


class MnsKernelStat(ctypes.Structure):
    _fields_ = [
        ("name", ctypes.c_char * 64),
        ("launches", ctypes.c_int64),
        ("ms", ctypes.c_double),
        ("flops", ctypes.c_double),
        ("bytes", ctypes.c_double),
    ]


class MnsError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {message} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it with "
            "`python -m muon_newton_schulz_amd.build` (or __graft_entry__.build()).")
    lib = ctypes.CDLL(path)
    sz = ctypes.POINTER(ctypes.c_size_t)
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    fp = ctypes.POINTER(ctypes.c_float)
    lib.mns_status_string.restype = ctypes.c_char_p
    lib.mns_status_string.argtypes = [ctypes.c_int]
    lib.mns_version.restype = ctypes.c_int
    lib.mns_version.argtypes = []
    lib.mns_step_workspace_size.restype = ctypes.c_int
    lib.mns_step_workspace_size.argtypes = [ctypes.POINTER(MnsMatrix), ctypes.c_int,
                                            ctypes.POINTER(MnsHparams), sz]
    lib.muon_step.restype = ctypes.c_int
    lib.muon_step.argtypes = [ctypes.POINTER(MnsMatrix), ctypes.c_int,
                              ctypes.POINTER(MnsHparams), vp, ctypes.c_size_t, vp]
    lib.mns_ns_workspace_size.restype = ctypes.c_int
    lib.mns_ns_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.c_int, sz]
    lib.ns_orthogonalize.restype = ctypes.c_int
    lib.ns_orthogonalize.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, fp,
                                     vp, ctypes.c_size_t, vp]
    lib.gram_ns_orthogonalize.restype = ctypes.c_int
    lib.gram_ns_orthogonalize.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, fp,
                                          ctypes.c_uint32, vp, ctypes.c_size_t, vp]
    lib.mns_normuon_workspace_size.restype = ctypes.c_int
    lib.mns_normuon_workspace_size.argtypes = [i64, i64, i64, sz]
    lib.normuon_scale.restype = ctypes.c_int
    lib.normuon_scale.argtypes = [vp, ctypes.c_int, i64, i64, i64, fp, ctypes.c_float,
                                  ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.mns_profile_begin.restype = ctypes.c_int
    lib.mns_profile_begin.argtypes = []
    lib.mns_profile_end.restype = ctypes.c_int
    lib.mns_profile_end.argtypes = [ctypes.POINTER(MnsKernelStat), ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_int)]
    lib.ns_orthogonalize_noalloc.restype = ctypes.c_int
    lib.ns_orthogonalize_noalloc.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int,
                                             fp, vp]
    lib.mns_profile_set_flush.restype = ctypes.c_int
    lib.mns_profile_set_flush.argtypes = [vp, ctypes.c_size_t]
    _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != MNS_OK:
        msg = load().mns_status_string(status).decode()
        raise MnsError(status, where, msg)
