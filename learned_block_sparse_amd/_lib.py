"""ctypes view of libveda (include/veda.h): structs, prototypes, loading.

Argument marshalling only; every step of the hot path runs in libveda's
kernels. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# VEDA_LIBRARY names another build of the library to load (the tests use it
# for the sanitizer build of the host-only entry points).
LIB_PATH = os.environ.get("VEDA_LIBRARY") or os.path.join(PKG, "libveda.so")

TILE = 128
MAX_SPANS = 16
MAX_BLOCKS = 2
MAX_HEADS = 256
STATIC_SCRATCH_BYTES = 64 << 20     # VEDA_STATIC_SCRATCH_BYTES

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_DEVICE = 0, 1, 2, 3
F32, BF16 = 0, 1

EXPORTS = ("veda_last_error", "veda_version", "veda_plan_query", "veda_plan",
           "veda_select_query", "veda_select", "veda_attend", "veda_attend_check",
           "veda_select_static", "veda_teacher", "veda_recall", "veda_attend_int8_query",
           "veda_attend_int8")


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


class _HostOnly:
    """A host-only build: prototypes of launching entry points are accepted
    and dropped; calling one raises."""

    def __init__(self, lib):
        object.__setattr__(self, "_l", lib)

    def __getattr__(self, name):
        if hasattr(self._l, name):
            return getattr(self._l, name)
        raise AttributeError(f"{name} is not in this host-only build of libveda")

    def __setattr__(self, name, value):
        setattr(self._l, name, value)


def has_kernels() -> bool:
    """Whether the loaded library holds the kernels and launching entry points."""
    return not isinstance(load(), _HostOnly)


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
    protos = {
        "veda_last_error": (C.c_char_p, []),
        "veda_version": (C.c_char_p, []),
        "veda_plan_query": (C.c_int, [C.POINTER(Span), I32, I64, C.POINTER(PlanInfo)]),
        "veda_plan": (C.c_int, [C.POINTER(PlanInfo), P, P, P]),
        "veda_select_query": (C.c_int, [C.POINTER(PlanInfo), Budget, Budget, I32, I32,
                                        C.POINTER(SelectInfo)]),
        "veda_select": (C.c_int, [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P,
                                  C.c_int, I64, I64, I32, C.POINTER(I32), P, P, P, P, P, I32, P,
                                  SZ, P]),
        "veda_attend": (C.c_int, [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P, P, P,
                                  C.c_int, I64, I64, I64, I64, I32, C.POINTER(I32), P, P, F, P]),
        "veda_select_static": (C.c_int, [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P,
                                         C.c_int, I64, I64, I32, C.POINTER(I32), P, P, P, P, P]),
        "veda_teacher": (C.c_int, [C.POINTER(PlanInfo), P, P, P, P, C.c_int, I64, I64, I32,
                                   C.POINTER(I32), I32, I32, F, P, P]),
        "veda_recall": (C.c_int, [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P, P]),
        "veda_attend_check": (C.c_int, [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P,
                                        P, P, C.c_int, I64, I64, I64, I64, I32, C.POINTER(I32),
                                        P, P]),
        "veda_attend_int8_query": (C.c_int, [C.POINTER(PlanInfo), C.POINTER(SelectInfo),
                                             C.POINTER(SZ)]),
        "veda_attend_int8": (C.c_int, [C.POINTER(PlanInfo), C.POINTER(SelectInfo), P, P, P, P, P,
                                       P, I64, I64, I64, I64, I32, C.POINTER(I32), P, P, F, P, SZ,
                                       P]),
    }
    for name, (res, args) in protos.items():
        if hasattr(lib, name):
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
    if not hasattr(lib, "veda_attend"):   # host-only build: no launching entry points
        lib = _HostOnly(lib)
    _lib = lib
    return lib
