"""ctypes binding of libskipln.so (the C ABI declared in include/skipln.h).

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the library.  There is no fallback: if the library cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libskipln.so")

# Values of the enums in include/skipln.h (a CPU test checks they match).
F32, F16 = 0, 1
SKIP_EXACT, SKIP_BROADCAST, SKIP_BROADCAST_INNER = 0, 1, 2
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_MODE, ERR_EPS, ERR_ALIAS = 0, 1, 2, 3, 4, 5, 6
ERR_UNSUPPORTED, ERR_LAUNCH, ERR_DEVICE, ERR_VARIANT, ERR_OP, ERR_WORKSPACE = 7, 8, 9, 10, 11, 12
OP_LAYER_NORM, OP_SIMPLIFIED, OP_BIAS_ADD, OP_BIAS_SOFTMAX = 0, 1, 2, 3
VARIANT_AUTO, VARIANT_GENERIC, VARIANT_ROWTILE, VARIANT_MULTIWAVE, VARIANT_LDSROW, VARIANT_SPLITROW = 0, 1, 2, 3, 4, 5
VARIANT_ELEMENT, VARIANT_REGROW = 6, 7
VARIANT_GEOMETRY, VARIANT_ELEMENT_GEOMETRY = 64, 128
TILE_CONTIGUOUS, TILE_STRIDED, TILE_SKIP_STATIONARY = 0, 1, 2

# Every function the header declares: name -> (restype, argtypes).
_vp, _i64, _i32, _f32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
SIGNATURES = {
    "skipln_forward": (_i32, [_vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _i32, _vp]),
    "skipln_forward_simplified": (_i32, [_vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _i32,
                                         _vp]),
    "skipln_bias_add": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp]),
    "skipln_bias_softmax": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _i64, _vp]),
    "skipln_forward_ws": (_i32, [_i32, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _i32, _i32,
                                 _vp, _i64, _vp]),
    "skipln_workspace_bytes": (_i64, [_i32, _i64, _i64, _i32, _i32, _i64, _i32]),
    "skipln_select_ws": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "skipln_forward_variant": (_i32, [_i32, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _i32,
                                      _i32, _vp]),
    "skipln_forward_config": (_i32, [_i32, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _i32,
                                     _i32, _i64, _i32, _vp]),
    "skipln_validate": (_i32, [_i32, _vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _i32]),
    "skipln_select": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "skipln_copy": (_i32, [_vp, _vp, _i64, _vp]),
    "skipln_stream": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i64, _i32, _vp]),
    "skipln_rowtile_geometries": (_i32, []),
    "skipln_element_geometries": (_i32, []),
    "skipln_kernel_name": (C.c_char_p, [_i32]),
    "skipln_status_string": (C.c_char_p, [_i32]),
    "skipln_version": (_i32, []),
}

_lock = threading.Lock()
_lib = None


class SkiplnError(RuntimeError):
    def __init__(self, status: int, where: str = "skipln"):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load() -> C.CDLL:
    """Load libskipln.so, building it first if it does not exist yet."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from . import build as _build

                _build.build()
            lib = C.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    try:
        return load().skipln_status_string(int(status)).decode()
    except OSError:
        return "libskipln unavailable"


def kernel_name(kernel_id: int) -> str:
    return load().skipln_kernel_name(int(kernel_id)).decode()


def check(status: int, where: str) -> None:
    if status != OK:
        raise SkiplnError(status, where)
