"""ctypes binding of libskipln.so (the operator's C ABI, include/skipln.h)
and of libskipln_tune.so (the same kernels' tuning, introspection and probe
ABI, include/skipln_tune.h).

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the libraries.  There is no fallback: if a library cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libskipln.so")
TUNE_LIB_PATH = os.path.join(PKG, "libskipln_tune.so")

# Values of the enums in include/skipln.h and include/skipln_tune.h (a CPU test
# checks they match).
F32, F16 = 0, 1
SKIP_EXACT, SKIP_BROADCAST, SKIP_BROADCAST_INNER = 0, 1, 2
OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_MODE, ERR_EPS, ERR_ALIAS = 0, 1, 2, 3, 4, 5, 6
ERR_UNSUPPORTED, ERR_LAUNCH, ERR_DEVICE, ERR_VARIANT, ERR_OP, ERR_WORKSPACE = 7, 8, 9, 10, 11, 12
OP_LAYER_NORM, OP_SIMPLIFIED, OP_BIAS_ADD, OP_BIAS_SOFTMAX = 0, 1, 2, 3
VARIANT_AUTO, VARIANT_GENERIC, VARIANT_ROWTILE, VARIANT_MULTIWAVE, VARIANT_LDSROW, VARIANT_SPLITROW = 0, 1, 2, 3, 4, 5
VARIANT_ELEMENT, VARIANT_REGROW, VARIANT_SPAN = 6, 7, 8
VARIANT_GEOMETRY, VARIANT_ELEMENT_GEOMETRY, VARIANT_SPAN_GEOMETRY = 64, 128, 192
TILE_CONTIGUOUS, TILE_STRIDED, TILE_SKIP_STATIONARY = 0, 1, 2
STORE_AUTO, STORE_STREAM, STORE_THROUGH = -1, 0, 1

# Every function each header declares: name -> (restype, argtypes).
_vp, _i64, _i32, _f32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
_FWD = [_vp, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _i32]  # input .. dtype
SIGNATURES = {
    "skipln_forward": (_i32, _FWD + [_vp]),
    "skipln_forward_simplified": (_i32, _FWD + [_vp]),
    "skipln_bias_add": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _vp]),
    "skipln_bias_softmax": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _i64, _vp]),
    "skipln_forward_ws": (_i32, [_i32] + _FWD + [_vp, _i64, _vp]),
    "skipln_forward_ws_static": (_i32, [_i32] + _FWD + [_vp]),
    "skipln_workspace_bytes": (_i64, [_i32, _i64, _i64, _i32, _i32, _i64]),
    "skipln_validate": (_i32, _FWD),
    "skipln_status_string": (C.c_char_p, [_i32]),
    "skipln_version": (_i32, []),
}
TUNE_SIGNATURES = {
    "skipln_tune_forward": (_i32, [_i32] + _FWD + [_i32, _vp, _i64, _vp]),
    "skipln_tune_forward_config": (_i32, [_i32] + _FWD + [_i32, _i64, _i32, _i32, _vp]),
    "skipln_tune_forward_form": (_i32, [_i32] + _FWD + [_i32, _i32, _i32, _i32, _vp]),
    "skipln_tune_blocks_per_cu": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "skipln_tune_workspace_bytes": (_i64, [_i32, _i64, _i64, _i32, _i32, _i64, _i32]),
    "skipln_tune_select": (_i32, [_i32, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32]),
    "skipln_tune_kernel_name": (C.c_char_p, [_i32]),
    "skipln_tune_rowtile_geometries": (_i32, []),
    "skipln_tune_element_geometries": (_i32, []),
    "skipln_tune_span_geometries": (_i32, []),
    "skipln_tune_validate": (_i32, [_i32] + _FWD),
    "skipln_tune_copy": (_i32, [_vp, _vp, _i64, _vp]),
    "skipln_tune_stream": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i64, _i32, _vp]),
}

_lock = threading.Lock()
_libs = {}


class SkiplnError(RuntimeError):
    """A status other than SKIPLN_OK; ``status`` holds the code."""

    def __init__(self, status: int, where: str = "skipln"):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


class SkiplnArgumentError(SkiplnError, ValueError):
    """A status that rejects the call's arguments (nothing was enqueued)."""


# Statuses that reject arguments; the others report the runtime or device.
ARGUMENT_STATUSES = frozenset({ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_MODE, ERR_EPS, ERR_ALIAS, ERR_UNSUPPORTED,
                               ERR_VARIANT, ERR_OP, ERR_WORKSPACE})


def _open(path: str, signatures) -> C.CDLL:
    if path not in _libs:
        # torch first: its HIP runtime (libamdhip64.so.7, bundled with the
        # wheel) then serves the library too, so kernels and tensors share one
        # runtime.  Loaded the other way round, torch can bring up a second
        # runtime whose device the library's calls do not see.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        with _lock:
            if path not in _libs:
                if not os.path.exists(path):
                    from . import build as _build

                    _build.build()
                lib = C.CDLL(path)
                for name, (res, args) in signatures.items():
                    fn = getattr(lib, name)
                    fn.restype = res
                    fn.argtypes = args
                _libs[path] = lib
    return _libs[path]


def load() -> C.CDLL:
    """The operator library, libskipln.so (built first if it does not exist)."""
    return _open(LIB_PATH, SIGNATURES)


def load_tune() -> C.CDLL:
    """The tuning library, libskipln_tune.so (built first if it does not exist)."""
    return _open(TUNE_LIB_PATH, TUNE_SIGNATURES)


def status_string(status: int) -> str:
    try:
        return load().skipln_status_string(int(status)).decode()
    except OSError:
        return "libskipln unavailable"


def kernel_name(kernel_id: int) -> str:
    return load_tune().skipln_tune_kernel_name(int(kernel_id)).decode()


def check(status: int, where: str) -> None:
    """Raise for any status but SKIPLN_OK: SkiplnArgumentError (also a
    ValueError) for rejected arguments, SkiplnError otherwise."""
    if status != OK:
        raise (SkiplnArgumentError if status in ARGUMENT_STATUSES else SkiplnError)(status, where)
