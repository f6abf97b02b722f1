"""ctypes binding of libmla_verify.so (the C ABI in include/mla_verify.h).

Argument marshalling only: tensors are checked and their device pointers and
the current HIP stream are handed to the library, which does all the work.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_verify.so")

MLAV_OK = 0
MLAV_ERR_NULL = 1
MLAV_ERR_SHAPE = 2
MLAV_ERR_TREE = 3
MLAV_ERR_ALIGN = 4
MLAV_ERR_WORKSPACE = 5
MLAV_ERR_UNSUPPORTED = 6
MLAV_ERR_HIP = 7
MLAV_ERR_ARG = 8
MLAV_ERR_SCRATCH = 9
MLAV_SCRATCH_BYTES = 24 << 20

# the functions include/mla_verify.h declares
EXPORTS = (
    "mla_verify",
    "mla_verify_ex",
    "mla_verify_noalloc",
    "mla_verify_batched",
    "mla_verify_paged",
    "mla_verify_partials",
    "mla_verify_workspace_size",
    "mla_verify_plan",
    "mla_verify_check_tree",
    "mla_verify_combine",
    "mla_verify_strerror",
)


class Options(ctypes.Structure):
    _fields_ = [("nsplit", c_int32), ("pv_mode", c_int32), ("kernel", c_int32), ("partials", c_int32),
                ("phase", c_int32), ("merge", c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("nsplit", c_int32), ("tile", c_int32), ("chunk", c_int64), ("grid", c_int32),
                ("combine", c_int32)]


class MLAVError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({strerror(status)})")
        self.status = status


_lib = None


def load():
    """Load the library once (works without a GPU; calls need one)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m mla_tree_verify_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    tensors = [c_void_p] * 4
    lib.mla_verify.argtypes = tensors + [c_void_p, c_int64, c_float, c_void_p, c_void_p, c_int32,
                                         c_int32, c_void_p, c_size_t, c_void_p]
    lib.mla_verify.restype = c_int32
    lib.mla_verify_ex.argtypes = lib.mla_verify.argtypes + [POINTER(Options)]
    lib.mla_verify_ex.restype = c_int32
    lib.mla_verify_noalloc.argtypes = tensors + [c_void_p, c_int64, c_float, c_void_p, c_void_p, c_int32,
                                                 c_int32, c_void_p, POINTER(Options)]
    lib.mla_verify_noalloc.restype = c_int32
    lib.mla_verify_batched.argtypes = tensors + [c_void_p, c_void_p, c_int32, c_int64, c_int64, c_float,
                                                 c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_size_t,
                                                 c_void_p, POINTER(Options)]
    lib.mla_verify_batched.restype = c_int32
    lib.mla_verify_paged.argtypes = tensors + [c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_int64, c_int64,
                                               c_float, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_size_t,
                                               c_void_p, POINTER(Options)]
    lib.mla_verify_paged.restype = c_int32
    lib.mla_verify_partials.argtypes = tensors + [c_void_p, c_int64, c_float, c_void_p, c_void_p, c_int32,
                                                  c_int32, POINTER(Plan), c_void_p, POINTER(Options)]
    lib.mla_verify_partials.restype = c_int32
    lib.mla_verify_workspace_size.argtypes = [c_int32, c_int32, c_int32, c_int64, c_int64, c_int32,
                                              POINTER(Options)]
    lib.mla_verify_workspace_size.restype = c_size_t
    lib.mla_verify_plan.argtypes = [c_int32, c_int32, c_int32, c_int64, c_int64, c_int32,
                                    POINTER(Options), POINTER(Plan)]
    lib.mla_verify_plan.restype = c_int32
    lib.mla_verify_check_tree.argtypes = [POINTER(c_int32), c_int32]
    lib.mla_verify_check_tree.restype = c_int32
    lib.mla_verify_combine.argtypes = [c_void_p, c_void_p, c_int32, c_int64, c_void_p, c_void_p, c_void_p]
    lib.mla_verify_combine.restype = c_int32
    lib.mla_verify_strerror.argtypes = [c_int32]
    lib.mla_verify_strerror.restype = c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().mla_verify_strerror(status).decode()


def options(nsplit: int = 0, pv_mode: int = 0, kernel: int = 0, partials: int = 0, phase: int = 0,
            merge: int = 0) -> Options:
    return Options(nsplit, pv_mode, kernel, partials, phase, merge)


def plan(q_len: int, num_heads: int, batch: int, total_kv: int, max_kv: int, num_cus: int,
         nsplit: int = 0, pv_mode: int = 0, kernel: int = 0, partials: int = 0, merge: int = 0) -> Plan:
    p = Plan()
    opt = options(nsplit, pv_mode, kernel, partials, merge=merge)
    rc = load().mla_verify_plan(q_len, num_heads, batch, total_kv, max_kv, num_cus, ctypes.byref(opt),
                                ctypes.byref(p))
    if rc != MLAV_OK:
        raise MLAVError(rc, "mla_verify_plan")
    return p


def workspace_size(q_len: int, num_heads: int, batch: int, total_kv: int, max_kv: int, num_cus: int = 0,
                   nsplit: int = 0, pv_mode: int = 0, kernel: int = 0, partials: int = 0, merge: int = 0) -> int:
    opt = options(nsplit, pv_mode, kernel, partials, merge=merge)
    return int(load().mla_verify_workspace_size(q_len, num_heads, batch, total_kv, max_kv, num_cus,
                                                 ctypes.byref(opt)))


def check_tree(parents) -> int:
    arr = (c_int32 * len(parents))(*[int(p) for p in parents])
    return int(load().mla_verify_check_tree(arr, len(parents)))
