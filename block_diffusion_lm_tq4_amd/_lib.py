"""ctypes loader for libtq4.so (the C ABI declared in include/tq4.h).

The library is built in-tree by ``block_diffusion_lm_tq4_amd.build``.  If it is
missing, every entry point raises: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

# TQ4_LIBRARY selects another build of the same library (for example the
# sanitizer build of block_diffusion_lm_tq4_amd.build.build_sanitized)
LIB_PATH = os.environ.get("TQ4_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libtq4.so")

TQ4_OK = 0
STATUS_NAMES = {
    0: "TQ4_OK",
    1: "TQ4_E_NULL",
    2: "TQ4_E_SHAPE",
    3: "TQ4_E_ALIGN",
    4: "TQ4_E_WORKSPACE",
    5: "TQ4_E_DEVICE",
    6: "TQ4_E_TOO_LARGE",
}

# every symbol include/tq4.h declares, with (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
SIGNATURES = {
    "tq4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tq4_version": (ctypes.c_int, []),
    "tq4_codebook": (ctypes.c_int, [_P]),
    "tq4_packed_size": (_SZ, [_I64, _I64]),
    "tq4_pack": (ctypes.c_int, [_P, _I64, _I64, _U32, _P, _P, _P]),
    "tq4_pack_bf16": (ctypes.c_int, [_P, _I64, _I64, _U32, _P, _P, _P]),
    "tq4_act_rht": (ctypes.c_int, [_P, _I64, _I64, _U32, _P, _P]),
    "tq4_linear_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "tq4_linear": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _U32, _P, _P, _SZ, _P]),
    "tq4_linear_epilogue": (ctypes.c_int,
                            [_P, _I64, _I64, _P, _I64, _U32, _P, _P, _P, _P, _SZ, _P]),
    "tq4_linear_epilogue_bf16": (ctypes.c_int,
                                 [_P, _I64, _I64, _P, _I64, _U32, _P, _P, _P, _P, _SZ, _P]),
    "tq4_fp8_cache_size": (ctypes.c_size_t, [_I64, _I64]),
    "tq4_fp8_cache": (ctypes.c_int, [_P, _I64, _I64, _U32, _P, _P]),
    "tq4_act_mxfp8": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "tq4_linear_fp8_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "tq4_linear_fp8": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _SZ, _P]),
    "tq4_linear_fp8_quantized": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, _P]),
    "tq4_moe_block_workspace_size": (ctypes.c_size_t, [_I64, _I32, _I32, _I64, _I64]),
    "tq4_moe_block": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _I32, _P, _I64, _P, _U32, _P, _P,
                                     _SZ, _P]),
    "tq4_moe_block_persistent_workspace_size": (ctypes.c_size_t, [_I64, _I32, _I32, _I64, _I64]),
    "tq4_moe_block_persistent": (ctypes.c_int, [_P, _I64, _I64, _P, _I32, _I32, _P, _I64, _P, _U32,
                                                _P, _P, _SZ, _P]),
    "tq4_linear_rotated": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P, _SZ, _P]),
    "tq4_linear_noalloc": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _U32, _P, _P]),
    "tq4_linear_variant": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _U32, _P, _P, _SZ,
                                          ctypes.c_int, _P]),
    "tq4_moe_route": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P]),
    "tq4_moe_workspace_size": (_SZ, [_I64, _I32, _I32, _I64, _I64]),
    "tq4_moe_grouped": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _P, _I64, _P, _U32,
                                       _P, _P, _SZ, _P]),
    "tq4_moe_grouped_fp8_workspace_size": (_SZ, [_I64, _I32, _I32, _I64, _I64]),
    "tq4_moe_grouped_fp8": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I32, _I32, _P, _I64, _P,
                                           _P, _P, _SZ, _P]),
    "tq4_moe_router": (ctypes.c_int, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "tq4_read_probe": (ctypes.c_int, [_P, _I64, _P, _P]),
}

_lock = threading.Lock()
_lib = None


class TQ4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn} failed: {name}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libtq4.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m block_diffusion_lm_tq4_amd.build` (no fallback path exists)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def check(fn: str, status: int) -> None:
    if status != TQ4_OK:
        raise TQ4Error(fn, status)
