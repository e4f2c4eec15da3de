"""ctypes front end of the C oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may call
this module.  It marshals numpy arrays into ``liboracle.so`` (built from
``skipln_oracle.c``) and returns binary64 results; see that file for the
definition it implements and where each step comes from.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

from . import build as _build

_LIBS = {}
_CODES = {np.dtype(np.float32): 0, np.dtype(np.float16): 1}
_CURRENT = None


def lib() -> C.CDLL:
    """The library in use: ``liboracle.so`` unless :func:`use` picked another
    build of the same source (the tests use that to run the pins against
    copies of the oracle with a planted mistake)."""
    global _CURRENT
    if _CURRENT is None:
        if not os.path.exists(_build.LIB):
            _build.build(force=True)
        _CURRENT = _load(_build.LIB)
    return _CURRENT


def use(path: Optional[str]) -> None:
    """Route every call of this module to the oracle library at ``path``
    (None: back to the default build)."""
    global _CURRENT
    _CURRENT = None if path is None else _load(path)


def _load(path: str) -> C.CDLL:
    if path not in _LIBS:
        L = C.CDLL(path)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        L.oracle_skip_norm.argtypes = [vp, vp, i64, vp, vp, vp, i32, i64, i64, i64,
                                       C.c_float, i32, vp, vp, vp, vp, i32]
        L.oracle_skip_norm.restype = i32
        L.oracle_bias_add.argtypes = [vp, vp, vp, i32, i64, i64, vp, vp]
        L.oracle_bias_add.restype = i32
        L.oracle_f16_to_f32_array.argtypes = [vp, vp, i64]
        L.oracle_f16_to_f32_array.restype = None
        L.oracle_f32_to_f16_array.argtypes = [vp, vp, i64]
        L.oracle_f32_to_f16_array.restype = None
        L.oracle_bias_softmax.argtypes = [vp, vp, i32, i64, i64, i64, i32, vp]
        L.oracle_bias_softmax.restype = i32
        L.oracle_version.restype = i32
        _LIBS[path] = L
    return _LIBS[path]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _code(*arrays) -> int:
    dts = {a.dtype for a in arrays if a is not None}
    if len(dts) != 1:
        raise TypeError(f"all tensors must share one dtype, got {dts}")
    dt = dts.pop()
    if dt not in _CODES:
        raise TypeError(f"unsupported dtype {dt}")
    return _CODES[dt]


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (uint16) -> binary32 values, by the oracle's converter."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib().oracle_f16_to_f32_array(_ptr(b), _ptr(out), b.size)
    return out


def f32_to_f16(values: np.ndarray) -> np.ndarray:
    """binary32 values -> binary16 bit patterns (uint16), round to nearest even."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_f32_to_f16_array(_ptr(v), _ptr(out), v.size)
    return out


def skip_layer_norm(
    x: np.ndarray,
    skip: np.ndarray,
    gamma: np.ndarray,
    beta: Optional[np.ndarray] = None,
    bias: Optional[np.ndarray] = None,
    eps: float = 1e-12,
    *,
    broadcast: bool = False,
    row_offset: int = 0,
    residual: bool = True,
    simplified: bool = False,
    stats: bool = False,
    threads: int = 1,
):
    """Reference forward pass over the rows of ``x`` (shape ``(rows, H)``).

    ``skip`` is ``(rows, H)`` (exact) or, with ``broadcast=True``, ``(S, H)``
    where logical row ``row_offset + i`` reads skip row
    ``(row_offset + i) mod S``.  Returns a dict with ``y`` (binary64, the
    unrounded normalized output), ``residual`` (the pre-normalization sum in
    the I/O type, or None) and, with ``stats=True``, per-row ``mean`` and
    ``var`` (binary64).
    """
    x = np.ascontiguousarray(x)
    skip = np.ascontiguousarray(skip)
    gamma = np.ascontiguousarray(gamma)
    beta = None if beta is None else np.ascontiguousarray(beta)
    bias = None if bias is None else np.ascontiguousarray(bias)
    code = _code(x, skip, gamma, beta, bias)
    if x.ndim != 2:
        raise ValueError("x must be (rows, H)")
    rows, h = x.shape
    if skip.ndim != 2 or skip.shape[1] != h:
        raise ValueError("skip must be (rows, H) or (S, H)")
    if not broadcast and skip.shape[0] != rows:
        raise ValueError("exact skip must have as many rows as x")
    for v in (gamma, beta, bias):
        if v is not None and v.shape != (h,):
            raise ValueError("gamma/beta/bias must have length H")
    y = np.empty((rows, h), dtype=np.float64)
    res = np.empty((rows, h), dtype=x.dtype) if residual else None
    mean = np.empty(rows, dtype=np.float64) if stats else None
    var = np.empty(rows, dtype=np.float64) if stats else None
    st = lib().oracle_skip_norm(
        _ptr(x), _ptr(skip), skip.shape[0] if broadcast else 0, _ptr(gamma), _ptr(beta),
        _ptr(bias), code, rows, h, row_offset, float(np.float32(eps)), int(simplified),
        _ptr(res), _ptr(y), _ptr(mean), _ptr(var), int(threads),
    )
    if st != 0:
        raise RuntimeError(f"oracle_skip_norm failed with status {st}")
    return {"y": y, "residual": res, "mean": mean, "var": var}


def bias_add(x: np.ndarray, bias: np.ndarray, skip: np.ndarray):
    """Reference BiasAdd: returns (Y in the I/O type, X + bias + skip in binary64)."""
    x = np.ascontiguousarray(x)
    skip = np.ascontiguousarray(skip)
    bias = np.ascontiguousarray(bias)
    code = _code(x, bias, skip)
    h = x.shape[-1]
    if skip.shape != x.shape or bias.shape != (h,):
        raise ValueError("skip must match X and bias must have length C")
    rows = x.size // h if h else 0
    y = np.empty(x.shape, dtype=x.dtype)
    ye = np.empty(x.shape, dtype=np.float64)
    st = lib().oracle_bias_add(_ptr(x), _ptr(bias), _ptr(skip), code, rows, h, _ptr(y), _ptr(ye))
    if st != 0:
        raise RuntimeError(f"oracle_bias_add failed with status {st}")
    return y, ye


def bias_softmax(data: np.ndarray, bias: np.ndarray, inner: bool) -> np.ndarray:
    """Reference BiasSoftmax over rows: ``data`` is (batch_count, block_size),
    ``bias`` (bias_rows, block_size) with bias_rows dividing batch_count; row r
    adds bias row r // (batch_count // bias_rows) (inner) or r % bias_rows
    (outer).  Returns the binary64 softmax of the binary32 sum."""
    data = np.ascontiguousarray(data)
    bias = np.ascontiguousarray(bias)
    code = _code(data, bias)
    if data.ndim != 2 or bias.ndim != 2 or bias.shape[1] != data.shape[1]:
        raise ValueError("data (rows, block) and bias (bias_rows, block) expected")
    y = np.empty(data.shape, dtype=np.float64)
    st = lib().oracle_bias_softmax(_ptr(data), _ptr(bias), code, data.shape[0], data.shape[1], bias.shape[0],
                                   int(bool(inner)), _ptr(y))
    if st != 0:
        raise RuntimeError(f"oracle_bias_softmax failed with status {st}")
    return y
