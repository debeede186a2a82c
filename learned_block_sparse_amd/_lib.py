"""ctypes view of libveda (include/veda.h): structs, prototypes, loading.

Argument marshalling only; every step of the hot path runs in libveda's
kernels. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libveda.so")

TILE = 128
MAX_SPANS = 16
MAX_BLOCKS = 2
MAX_HEADS = 256

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_DEVICE = 0, 1, 2, 3
F32, BF16 = 0, 1

EXPORTS = ("veda_last_error", "veda_version", "veda_plan_query", "veda_plan",
           "veda_select_query", "veda_select", "veda_attend")


class Span(C.Structure):
    _fields_ = [("start", C.c_int64), ("grid", C.c_int32 * 3), ("shape", C.c_int32 * 3)]


class Budget(C.Structure):
    _fields_ = [("ratio", C.c_double), ("tiles", C.c_double)]


class PlanInfo(C.Structure):
    _fields_ = [("seq_len", C.c_int64), ("n_slots", C.c_int64), ("ref_tokens", C.c_int64),
                ("target_tokens", C.c_int64), ("global_rows", C.c_int64),
                ("n_tiles", C.c_int32), ("n_video", C.c_int32), ("n_ref", C.c_int32),
                ("n_global", C.c_int32), ("n_spans", C.c_int32), ("_pad", C.c_int32),
                ("spans", Span * MAX_SPANS), ("span_tile0", C.c_int32 * (MAX_SPANS + 1))]


class Block(C.Structure):
    _fields_ = [("start", C.c_int32), ("stop", C.c_int32), ("keep_all", C.c_int32),
                ("k_lo", C.c_int32), ("k_hi", C.c_int32), ("_pad", C.c_int32),
                ("frac", C.c_double)]


class SelectInfo(C.Structure):
    _fields_ = [("n_blocks", C.c_int32), ("head_dim", C.c_int32), ("n_heads", C.c_int32),
                ("widest", C.c_int32), ("entries_per_head", C.c_int64),
                ("workspace_bytes", C.c_size_t), ("blocks", Block * MAX_BLOCKS)]


_lib = None


def load():
    """The loaded libveda (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libveda.so not found at {LIB_PATH}: build it with "
            "`python -m learned_block_sparse_amd.build` (there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, D, F, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_double, C.c_float, C.c_size_t
    lib.veda_last_error.restype = C.c_char_p
    lib.veda_last_error.argtypes = []
    lib.veda_version.restype = C.c_char_p
    lib.veda_version.argtypes = []
    lib.veda_plan_query.restype = C.c_int
    lib.veda_plan_query.argtypes = [C.POINTER(Span), I32, I64, C.POINTER(PlanInfo)]
    lib.veda_plan.restype = C.c_int
    lib.veda_plan.argtypes = [C.POINTER(PlanInfo), P, P, P]
    lib.veda_select_query.restype = C.c_int
    lib.veda_select_query.argtypes = [C.POINTER(PlanInfo), Budget, Budget, I32, I32,
                                      C.POINTER(SelectInfo)]
    lib.veda_select.restype = C.c_int
    lib.veda_select.argtypes = [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P, C.c_int,
                                I64, I64, I32, C.POINTER(I32), P, P, P, P, P, I32, P, SZ, P]
    lib.veda_attend.restype = C.c_int
    lib.veda_attend.argtypes = [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P, P, P,
                                C.c_int, I64, I64, I64, I64, I32, C.POINTER(I32), P, P, F, P]
    _lib = lib
    return lib
