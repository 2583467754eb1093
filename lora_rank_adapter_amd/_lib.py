"""ctypes view of the C ABI declared in include/lora.h.

Loads the in-tree ``liblora_mi355x.so``; if it is missing, or was built from
other sources than the ones in the tree (the build records a digest of them),
it is built first (hipcc). There is no other implementation behind these
calls: when the library cannot be built or loaded, every op raises.
"""
from __future__ import annotations

import ctypes
import threading

from . import build as _build

LORA_F32 = 0
LORA_BF16 = 1

LORA_OP_FWD = 0
LORA_OP_BWD_DX_DA = 1
LORA_OP_BWD_DB = 2

STATUS = {
    0: "LORA_OK",
    -1: "LORA_ERR_NULL",
    -2: "LORA_ERR_SHAPE",
    -3: "LORA_ERR_DTYPE",
    -4: "LORA_ERR_STRIDE",
    -5: "LORA_ERR_RANK",
    -6: "LORA_ERR_WORKSPACE",
    -7: "LORA_ERR_LAUNCH",
    -8: "LORA_ERR_LIMIT",
}


class LoraMat(ctypes.Structure):
    _fields_ = [
        ("ptr", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("stride_row", ctypes.c_int64),
        ("stride_col", ctypes.c_int64),
    ]


class LoraT3(ctypes.Structure):
    _fields_ = [
        ("ptr", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("d0", ctypes.c_int64),
        ("d1", ctypes.c_int64),
        ("d2", ctypes.c_int64),
        ("s0", ctypes.c_int64),
        ("s1", ctypes.c_int64),
        ("s2", ctypes.c_int64),
    ]


class LoraAddressing(ctypes.Structure):
    _fields_ = [
        ("token_slot", ctypes.c_void_p),
        ("T", ctypes.c_int32),
        ("S", ctypes.c_int32),
        ("counts", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("sorted_tokens", ctypes.c_void_p),
    ]


# exported symbol -> (restype, argtypes)
_P = ctypes.POINTER
SIGNATURES = {
    "lora_abi_version": (ctypes.c_int, []),
    "lora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "lora_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.c_int32]),
    "lora_fwd": (ctypes.c_int, [_P(LoraMat), _P(LoraMat), _P(LoraMat), _P(LoraMat), ctypes.c_float,
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "lora_bwd_dx_da": (ctypes.c_int, [_P(LoraMat), _P(LoraMat), _P(LoraMat), _P(LoraMat), ctypes.c_float,
                                      _P(LoraMat), _P(LoraMat), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "lora_bwd_dx_da_accumulate": (ctypes.c_int, [_P(LoraMat), _P(LoraMat), _P(LoraMat), _P(LoraMat),
                                                 ctypes.c_float, _P(LoraMat), _P(LoraMat), ctypes.c_void_p,
                                                 ctypes.c_size_t, ctypes.c_void_p]),
    "lora_bwd_db": (ctypes.c_int, [_P(LoraMat), _P(LoraMat), _P(LoraMat), ctypes.c_float, _P(LoraMat),
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "lora_addressing_build": (ctypes.c_int, [_P(LoraAddressing), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "lora_shrink": (ctypes.c_int, [_P(LoraMat), _P(LoraT3), _P(LoraAddressing), ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_int32, _P(LoraT3), ctypes.c_void_p]),
    "lora_expand_fused": (ctypes.c_int, [_P(LoraT3), _P(LoraT3), _P(LoraAddressing), ctypes.c_void_p,
                                         ctypes.c_void_p, _P(LoraMat), _P(ctypes.c_int64), ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p]),
    "lora_apply_linear": (ctypes.c_int, [_P(LoraMat), _P(LoraT3), _P(LoraT3), _P(LoraAddressing), ctypes.c_void_p,
                                         ctypes.c_void_p, _P(LoraMat), _P(ctypes.c_int64), ctypes.c_int32,
                                         ctypes.c_int32, _P(LoraT3), ctypes.c_void_p]),
    "lora_apply_linear_noalloc": (ctypes.c_int, [_P(LoraMat), _P(LoraT3), _P(LoraT3), _P(LoraAddressing),
                                                 ctypes.c_void_p, ctypes.c_void_p, _P(LoraMat), _P(ctypes.c_int64),
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "lora_gather_shrink": (ctypes.c_int, [ctypes.c_void_p, _P(LoraT3), _P(LoraAddressing), ctypes.c_void_p,
                                          ctypes.c_int32, _P(LoraT3), ctypes.c_void_p]),
    "lora_timing_begin": (ctypes.c_int, []),
    "lora_timing_pause": (ctypes.c_int, []),
    "lora_timing_resume": (ctypes.c_int, []),
    "lora_timing_read": (ctypes.c_int, [_P(ctypes.c_double), _P(ctypes.c_int64)]),
    "lora_timing_reserve": (ctypes.c_int, [ctypes.c_int64]),
}

_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _build.LIB_PATH


def load() -> ctypes.CDLL:
    """Load the HIP library (building it first when it is absent or stale) and
    bind every symbol."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _build.is_stale():
            _build.build()
        lib = ctypes.CDLL(_build.LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, '?')})")


def check(fn: str, status: int) -> None:
    if status != 0:
        raise LoraError(fn, status)
