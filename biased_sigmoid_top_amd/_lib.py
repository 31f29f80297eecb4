"""ctypes binding of liblfm_moe.so: argument marshalling only.

Every step of the layer runs in the library's HIP kernels.  When the library
is missing or cannot be loaded this module raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblfm_moe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "lfm_moe.h")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_WORKSPACE_TOO_SMALL = 2
ERR_OUT_OF_MEMORY = 3
ERR_HIP = 4

(WS_IDX, WS_W, WS_BLOCKCOUNTS, WS_OFFSETS, WS_ROW2SLOT, WS_H, WS_Y, WS_X, WS_ROUTER_PARTIAL,
 WS_XQ, WS_XS, WS_HQ, WS_HS) = range(13)
DECODE_MAX_TOKENS = 4
FP8_MAX_TOKENS = 1 << 24
FP8_STREAM_TOKENS = 4
NOALLOC_MAX_TOKENS = 256
NOALLOC_SCRATCH_BYTES = 16 << 20

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "lfm_moe_abi_version": (ctypes.c_int, []),
    "lfm_moe_last_error": (ctypes.c_char_p, []),
    "lfm_moe_rmsnorm": (ctypes.c_int, [_P, _P, _I64, _P]),
    "lfm_moe_route": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P]),
    "lfm_moe_route_workspace_bytes": (_SZ, [_I64]),
    "lfm_moe_route_ws": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_pack_gateup_stacked": (ctypes.c_int, [_P, _P, _P]),
    "lfm_moe_pack_fp8_gateup_stacked": (ctypes.c_int, [_P, _P, _P, _P]),
    "lfm_moe_pack_gateup": (ctypes.c_int, [_P, _P, _P, _P]),
    "lfm_moe_pack_down": (ctypes.c_int, [_P, _P, _P]),
    "lfm_moe_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P]),
    "lfm_moe_workspace_bytes": (_SZ, [_I64]),
    "lfm_moe_workspace_offset": (_SZ, [_I64, ctypes.c_int]),
    "lfm_moe_forward_ws": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P]),
    "lfm_moe_experts_ws": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_block_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P]),
    "lfm_moe_block_forward_ws": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_stack_forward_ws": (ctypes.c_int, [_P, _P, ctypes.c_int, _I64, _P, _SZ, _P]),
    "lfm_moe_stage_dispatch": (ctypes.c_int, [_P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_stage_gateup": (ctypes.c_int, [_P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_stage_down": (ctypes.c_int, [_P, _I64, _P, _SZ, _P]),
    "lfm_moe_stage_combine": (ctypes.c_int, [_P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_pack_fp8_gateup": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "lfm_moe_pack_fp8_down": (ctypes.c_int, [_P, _P, _P, _P]),
    "lfm_moe_forward_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _P]),
    "lfm_moe_forward_fp8_ws": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_experts_fp8_ws": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "lfm_moe_release": (None, []),
    "lfm_moe_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "lfm_moe_timing_read": (ctypes.c_int, [_P, _P]),
}

class BlockWeights(ctypes.Structure):
    """lfm_moe_block_weights: one block's device weight pointers."""
    _fields_ = [("W_r", _P), ("bias", _P), ("W_gateup", _P), ("W_down", _P)]


STAGES = ("rmsnorm", "route", "dispatch", "gateup", "down", "combine")


class LfmMoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Loads the built library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python __graft_entry__.py build` "
            "(hipcc, gfx950).  There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def declared_functions(header: str = HEADER) -> list[str]:
    """Names of the functions include/lfm_moe.h declares."""
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lfm_moe_\w+)\s*\(", text)))


def check(fn: str, status: int) -> None:
    if status != OK:
        msg = load().lfm_moe_last_error()
        raise LfmMoeError(fn, status, msg.decode() if msg else "")


def call(fn: str, *args) -> int:
    """Calls a library function and raises on a non-OK status."""
    st = getattr(load(), fn)(*args)
    check(fn, st)
    return st
