"""ctypes declarations of the libmuon.so C ABI (include/muon.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmuon.so")

MUON_BF16, MUON_FP32 = 0, 1
MUON_OK, MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED, MUON_ERR_WORKSPACE, MUON_ERR_HIP = 0, -1, -2, -3, -4
MUON_MAX_STEPS = 64
MUON_WORKSPACE_ALIGN = 256
MUON_PTR_ALIGN = 16
MUON_STATIC_SCRATCH_BYTES = 256 << 20
KERNEL_KINDS = ("prep", "norm", "gram", "poly", "update", "final", "normuon", "apply",
                "gramq")

# Every symbol include/muon.h declares.
EXPORTS = (
    "muon_status_string",
    "muon_orthogonalize_workspace_bytes",
    "muon_step_workspace_bytes",
    "muon_plan_groups",
    "muon_orthogonalize",
    "muon_step",
    "muon_step_ex_workspace_bytes",
    "muon_step_ex",
    "muon_step_static",
    "muon_timing_enable",
    "muon_timing_read",
    "muon_probe_mfma_bf16",
    "muon_probe_copy",
)


class MuonCoeff(ctypes.Structure):
    _fields_ = [("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float)]


class MuonOptions(ctypes.Structure):
    _fields_ = [("weight_decay", ctypes.c_float), ("cautious", ctypes.c_int),
                ("normuon", ctypes.c_int), ("beta2", ctypes.c_float),
                ("normuon_eps", ctypes.c_float)]


class MuonTimingRecord(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("m", ctypes.c_int), ("n", ctypes.c_int),
                ("batch", ctypes.c_int), ("step", ctypes.c_int), ("ms", ctypes.c_float),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double),
                ("exec_flops", ctypes.c_double)]


_c_int_p = ctypes.POINTER(ctypes.c_int)
_vp = ctypes.c_void_p
_lib = None


def load() -> ctypes.CDLL:
    """Load libmuon.so (built in-tree).  Raises ImportError if it is missing:
    there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m muon_newton_schulz_step_amd.build` "
            "(hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.muon_status_string.argtypes = [ctypes.c_int]
    lib.muon_status_string.restype = ctypes.c_char_p
    lib.muon_orthogonalize_workspace_bytes.argtypes = [ctypes.c_int] * 4
    lib.muon_orthogonalize_workspace_bytes.restype = ctypes.c_size_t
    lib.muon_step_workspace_bytes.argtypes = [ctypes.c_int, _c_int_p, _c_int_p, ctypes.c_int]
    lib.muon_step_workspace_bytes.restype = ctypes.c_size_t
    lib.muon_plan_groups.argtypes = [ctypes.c_int, _c_int_p, _c_int_p, _c_int_p, _c_int_p,
                                     _c_int_p, _c_int_p, _c_int_p]
    lib.muon_plan_groups.restype = ctypes.c_int
    lib.muon_orthogonalize.argtypes = [
        _vp, ctypes.c_int, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_longlong, ctypes.POINTER(MuonCoeff), ctypes.c_int, ctypes.c_float,
        ctypes.c_int, _vp, ctypes.c_size_t, _vp]
    lib.muon_orthogonalize.restype = ctypes.c_int
    lib.muon_step.argtypes = [
        ctypes.c_int, _c_int_p, _c_int_p, ctypes.POINTER(_vp), ctypes.c_int,
        ctypes.POINTER(_vp), ctypes.c_int, ctypes.POINTER(_vp), ctypes.c_float,
        ctypes.c_float, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(MuonCoeff),
        ctypes.c_int, ctypes.c_float, ctypes.c_int, _vp, ctypes.c_size_t, _vp]
    lib.muon_step.restype = ctypes.c_int
    lib.muon_step_ex_workspace_bytes.argtypes = [ctypes.c_int, _c_int_p, _c_int_p, ctypes.c_int,
                                                 ctypes.POINTER(MuonOptions)]
    lib.muon_step_ex_workspace_bytes.restype = ctypes.c_size_t
    lib.muon_step_ex.argtypes = [
        ctypes.c_int, _c_int_p, _c_int_p, ctypes.POINTER(_vp), ctypes.c_int,
        ctypes.POINTER(_vp), ctypes.c_int, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
        ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_float),
        ctypes.POINTER(MuonCoeff), ctypes.c_int, ctypes.c_float, ctypes.c_int,
        ctypes.POINTER(MuonOptions), _vp, ctypes.c_size_t, _vp]
    lib.muon_step_ex.restype = ctypes.c_int
    lib.muon_step_static.argtypes = [
        ctypes.c_int, _c_int_p, _c_int_p, ctypes.POINTER(_vp), ctypes.c_int,
        ctypes.POINTER(_vp), ctypes.c_int, ctypes.POINTER(_vp), ctypes.c_float,
        ctypes.c_float, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(MuonCoeff),
        ctypes.c_int, ctypes.c_float, ctypes.c_int, _vp]
    lib.muon_step_static.restype = ctypes.c_int
    lib.muon_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp]
    lib.muon_probe_mfma_bf16.restype = ctypes.c_int
    lib.muon_probe_copy.argtypes = [_vp, _vp, ctypes.c_size_t, ctypes.c_int, _vp]
    lib.muon_probe_copy.restype = ctypes.c_int
    lib.muon_timing_enable.argtypes = [ctypes.c_int]
    lib.muon_timing_enable.restype = ctypes.c_int
    lib.muon_timing_read.argtypes = [ctypes.POINTER(MuonTimingRecord), ctypes.c_int, _c_int_p]
    lib.muon_timing_read.restype = ctypes.c_int
    _lib = lib
    return lib


def int_array(values):
    values = list(values)
    return (ctypes.c_int * max(1, len(values)))(*values)


def ptr_array(values):
    values = list(values)
    return (_vp * max(1, len(values)))(*values)


def float_array(values):
    values = list(values)
    return (ctypes.c_float * max(1, len(values)))(*values)


def coeff_array(coeffs):
    coeffs = [tuple(map(float, c)) for c in coeffs]
    arr = (MuonCoeff * max(1, len(coeffs)))()
    for i, (a, b, c) in enumerate(coeffs):
        arr[i].a, arr[i].b, arr[i].c = a, b, c
    return arr
