"""ctypes binding of liblrmoe.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module converts
torch tensors to device pointers and host arrays to the C structs the ABI
(``include/lrmoe.h``) declares. It raises if the library is missing: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrmoe.so")

OK, ERR_INVALID_ARG, ERR_INFEASIBLE_QUOTA, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(6)
F32, BF16 = 0, 1
COMPACT_PHYSICAL, COMPACT_ZERO_MASKED = 0, 1
SCATTER_TOKEN, SCATTER_SLOT, SCATTER_TOKEN_BESIDE = 0, 1, 2

EXPORTS = ("lrmoe_status_string", "lrmoe_version", "lrmoe_validate", "lrmoe_workspace_size",
           "lrmoe_backward_bytes", "lrmoe_plan_quotas", "lrmoe_score", "lrmoe_score_criterion", "lrmoe_select",
           "lrmoe_compact", "lrmoe_grouped_gemm_bwd", "lrmoe_scatter", "lrmoe_expert_forward",
           "lrmoe_select_noalloc", "lrmoe_compact_weighted", "lrmoe_grouped_gemm_bwd_gathered")


class LrmoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class InfeasibleQuotaError(LrmoeError):
    pass


class CProblem(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("T", ctypes.c_int32), ("K", ctypes.c_int32),
                ("D", ctypes.c_int32), ("F", ctypes.c_int32), ("swiglu", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32), ("N", ctypes.c_int64),
                ("seg_off", ctypes.POINTER(ctypes.c_int64)), ("quota", ctypes.POINTER(ctypes.c_int32))]


_lib = None


def load() -> ctypes.CDLL:
    """Load liblrmoe.so from the package directory (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER(CProblem)
    lib.lrmoe_status_string.restype = ctypes.c_char_p
    lib.lrmoe_status_string.argtypes = [ctypes.c_int]
    lib.lrmoe_version.restype = ctypes.c_char_p
    lib.lrmoe_version.argtypes = []
    sigs = {
        "lrmoe_validate": [P, ctypes.POINTER(i64), ctypes.POINTER(i64)],
        "lrmoe_workspace_size": [P, ctypes.c_int, ctypes.POINTER(sz)],
        "lrmoe_backward_bytes": [P, i32, ctypes.POINTER(sz)],
        "lrmoe_plan_quotas": [P, ctypes.POINTER(i32), ctypes.POINTER(i32), i32, i32, sz, ctypes.POINTER(i32),
                              ctypes.POINTER(i32), ctypes.POINTER(sz)],
        "lrmoe_score": [P, vp, vp, vp, vp, vp, vp, sz, vp],
        "lrmoe_score_criterion": [P, i32, vp, vp, vp, vp, vp, vp, sz, vp],
        "lrmoe_select": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "lrmoe_select_noalloc": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "lrmoe_compact": [P, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                          ctypes.c_size_t, vp],
        "lrmoe_grouped_gemm_bwd": [P, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                   sz, vp, vp],
        "lrmoe_compact_weighted": [P, vp, vp, vp, vp, vp],
        "lrmoe_grouped_gemm_bwd_gathered": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz,
                                            vp, vp],
        "lrmoe_scatter": [P, ctypes.c_int, i64, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
        "lrmoe_expert_forward": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().lrmoe_status_string(status).decode()


def check(status: int, where: str):
    if status == OK:
        return
    if status == ERR_INFEASIBLE_QUOTA:
        raise InfeasibleQuotaError(status, where)
    raise LrmoeError(status, where)


def make_problem_struct(E, T, K, D, F, swiglu, dtype, seg_off, quota):
    """Returns (CProblem, keepalive) with host copies of the offsets and quotas."""
    seg = np.ascontiguousarray(seg_off, dtype=np.int64)
    q = np.ascontiguousarray(quota, dtype=np.int32)
    if len(seg) != E + 1 or len(q) != E:
        raise ValueError("seg_off must have E+1 entries and quota E entries")
    p = CProblem(E=E, T=T, K=K, D=D, F=F, swiglu=int(bool(swiglu)), dtype=dtype, reserved=0,
                 N=int(seg[-1]),
                 seg_off=seg.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                 quota=q.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return p, (seg, q)
