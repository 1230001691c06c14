"""ctypes view of include/gdn.h (structs, status codes, prototypes).

Loading fails loudly when libgdn.so has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gdn.h")

GDN_OK = 0
GDN_E_NULL = -1
GDN_E_SHAPE = -2
GDN_E_HEADS = -3
GDN_E_UNSUPPORTED = -4
GDN_E_SLOT = -5
GDN_E_OVERLAP = -6
GDN_E_SEQLENS = -7
GDN_E_SCRATCH = -8
GDN_E_HIP = -9
GDN_E_ALIGN = -10

GDN_F32 = 0
GDN_BF16 = 1


class gdn_geometry(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
                ("conv_kernel", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("l2norm_eps", ctypes.c_float), ("rmsnorm_eps", ctypes.c_float),
                ("scale", ctypes.c_float)]


class gdn_layer_weights(ctypes.Structure):
    _fields_ = [("conv_weight", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p)]


class gdn_state_pool(ctypes.Structure):
    _fields_ = [("recurrent", ctypes.c_void_p), ("conv", ctypes.c_void_p),
                ("num_slots", ctypes.c_int32)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class gdn_linear_out(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("N", ctypes.c_int32), ("ldy", ctypes.c_int32)]


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_GP = ctypes.POINTER(gdn_geometry)
_WP = ctypes.POINTER(gdn_layer_weights)
_PP = ctypes.POINTER(gdn_state_pool)
_SZP = ctypes.POINTER(ctypes.c_size_t)

PROTOTYPES = {
    "gdn_abi_version": (ctypes.c_int, []),
    "gdn_last_error": (ctypes.c_char_p, []),
    "gdn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "gdn_slot_bytes": (ctypes.c_int, [_GP, _SZP, _SZP]),
    "gdn_prefill_scratch_bytes": (ctypes.c_int, [_GP, _I32, _I32, _SZP]),
    "gdn_conv_update": (ctypes.c_int, [_GP, _WP, _PP, _P, _P, _I32, _P, _P, _P]),
    "gdn_decode_batch": (ctypes.c_int, [_GP, _WP, _PP, _P, _P, _I32, _P, _P, _P, _P, _P,
                                        _P, _P]),
    "gdn_decode_workspace_bytes": (ctypes.c_int, [_GP, _I32, _SZP]),
    "gdn_decode_step": (ctypes.c_int, [_GP, _WP, _PP, _P, _P, _I32, _P, _P, _P, _P, _P, _P,
                                       _P, ctypes.c_size_t, _P]),
    "gdn_decode_step_noalloc": (ctypes.c_int, [_GP, _WP, _PP, _P, _P, _I32, _P, _P, _P, _P, _P,
                                               _P, _P]),
    "gdn_prefill_chunked": (ctypes.c_int, [_GP, _WP, _PP, _P, _P, _P, _P, _P, _I32, _P, _P,
                                           _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "gdn_linear": (ctypes.c_int, [_P, _I32, _I32, _I32, ctypes.POINTER(gdn_linear_out), _I32,
                                  _P]),
    "gdn_check_slots": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "gdn_state_compact": (ctypes.c_int, [_GP, _PP, _I32, _P, _P, _P, _P, _I32, _P]),
}


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m linear_attention_causal_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != GDN_OK:
        lib = load()
        msg = lib.gdn_last_error().decode() or lib.gdn_status_str(status).decode()
        raise GdnError(status, msg)


def header_functions() -> list[str]:
    """Names of the functions include/gdn.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, re.M)))
