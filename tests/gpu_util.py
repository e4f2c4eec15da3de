"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, compare with the oracle.

Tolerances: the normalized output is compared with the oracle's unrounded
binary64 value, |out - y| <= atol + rtol * |y| with (1e-5, 1e-5) for float32
and (2e-3, 2e-3) for float16; the residual (input_skip_bias_sum) must match
bit for bit; BiasAdd's output bit for bit.

BiasSoftmax (SOFTMAX_TOL): the kernels form the same binary32 z = data + bias
and maximum M as the oracle; each exponential 2^t, t = (z - M) log2 e, has a
relative error of about |t| 9.2e-8 (three binary32 roundings in t) plus
1.2e-7 (the exp2 instruction), the binary32 sum at most depth x 6e-8 (about
4e-6 for the longest per-lane chains here), the scaling 1.2e-7.  The
register-resident long-row kernel sums relative to a running per-lane
maximum and rescales its partial sum when the maximum grows: at most 16
rescales per lane, each an exp2 and a product (about 1.8e-7 each), adding
at most 2.9e-6 to the sum's error.  For every y >= 1e-20 (|t| <= 67) the
total stays below 1.3e-5: float32 uses rtol 2e-5 and
atol 1e-20 (smaller values, and results flushed below the binary32 normal
range).  float16 adds one rounding to nearest (2^-11 relative, at most 2^-25
absolute among subnormals): rtol 1e-3, atol 2^-24.  With float16 outputs the
register-resident kernel takes 1/S into the exponent, 2^(t - log2 S): at most
|log2 S| 1.2e-7 more (S <= the row's length < 2^20: 2.4e-6), still far below
the output's rounding.
"""
from __future__ import annotations

import sys
from typing import Optional

import numpy as np

import transformer_residual_add_amd as T
from transformer_residual_add_amd import _lib as L
from oracle import oracle as O

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 2e-3)}
SOFTMAX_TOL = {"f32": (1e-20, 2e-5), "f16": (2.0 ** -24, 1e-3)}
OPS = {"layer_norm": L.OP_LAYER_NORM, "simplified": L.OP_SIMPLIFIED, "bias_add": L.OP_BIAS_ADD,
       "bias_softmax": L.OP_BIAS_SOFTMAX}


def skip_mode(w) -> int:
    """The ABI's skip form for a workload."""
    if not w.broadcast:
        return L.SKIP_EXACT
    return L.SKIP_BROADCAST_INNER if w.inner else L.SKIP_BROADCAST


def torch_dtype(dt: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16}[dt]


def select(op: int, hidden: int, code: int, mode: int = L.SKIP_EXACT, aligned: int = 1,
           variant: int = L.VARIANT_AUTO, workspace: int = 0, rows: int = -1) -> int:
    """Kernel id the tuning library's choice gives for a call on the current
    device (negative: a status)."""
    return L.load_tune().skipln_tune_select(op, rows, hidden, code, mode, aligned, variant, workspace, 0)


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceCase:
    """Device copies of one workload's inputs and its output buffers.

    ``offset_elems`` shifts every tensor by that many elements inside a
    larger allocation (misaligned pointers)."""

    def __init__(self, w, inputs, residual: bool, offset_elems: int = 0, device: str = "cuda"):
        import torch

        self.w = w
        self.inputs = inputs
        dt = torch_dtype(w.dtype)
        self._keep = []

        def up(a: Optional[np.ndarray]):
            if a is None:
                return None
            t = torch.from_numpy(np.ascontiguousarray(a).reshape(-1))
            if offset_elems:
                buf = torch.empty(t.numel() + offset_elems, dtype=dt, device=device)
                buf[offset_elems:].copy_(t.to(device))
                self._keep.append(buf)
                return buf[offset_elems:]
            return t.to(device)

        def empty(n):
            buf = torch.full((n + offset_elems,), float("nan"), dtype=dt, device=device)
            self._keep.append(buf)
            return buf[offset_elems:]

        n = w.rows * w.hidden
        self.x = up(inputs["input"])
        self.skip = up(inputs["skip"])
        self.gamma = up(inputs["gamma"])
        self.beta = up(inputs["beta"])
        self.bias = up(inputs["bias"])
        self.out = empty(n)
        self.res = empty(n) if residual else None

    def workspace(self, variant: int = L.VARIANT_AUTO):
        """(pointer, bytes) of a fresh device workspace for ``skipln_forward_ws``."""
        import torch

        w = self.w
        n = T.workspace_bytes(OPS[w.op], w.rows, w.hidden, L.F32 if w.dtype == "f32" else L.F16, skip_mode(w),
                              w.skip_rows if w.broadcast else 0, variant)
        buf = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
        self._keep.append(buf)
        return buf.data_ptr(), n

    def run(self, variant: int = L.VARIANT_AUTO, stream: int = 0, out=None, res="default", workspace=None):
        """``workspace``: None (no workspace: the operation's own entry point,
        or skipln_tune_forward for a forced family), True (a fresh one of the
        size the call needs) or (pointer, bytes)."""
        w = self.w
        p = lambda t: None if t is None else t.data_ptr()
        o = self.out if out is None else out
        r = self.res if res == "default" else res
        if workspace is True:
            workspace = self.workspace(variant)
        T.forward_raw(p(self.x), p(self.skip), skip_mode(w), w.skip_rows if w.broadcast else 0, p(self.gamma),
                      p(self.beta), p(self.bias), p(o), p(r), w.rows, w.hidden, float(np.float32(w.eps)),
                      L.F32 if w.dtype == "f32" else L.F16, stream, variant, OPS[w.op], workspace=workspace)

    def run_config(self, geometry: int, tiles_per_block: int, strided: int, stream: int = 0,
                   store: int = L.STORE_AUTO):
        w = self.w
        p = lambda t: None if t is None else t.data_ptr()
        st = L.load_tune().skipln_tune_forward_config(
            OPS[w.op], p(self.x), p(self.skip), skip_mode(w), w.skip_rows if w.broadcast else 0, p(self.gamma),
            p(self.beta), p(self.bias), p(self.out), p(self.res), w.rows, w.hidden, float(np.float32(w.eps)),
            L.F32 if w.dtype == "f32" else L.F16, geometry, tiles_per_block, strided, store, stream or None)
        L.check(st, "skipln_tune_forward_config")

    def run_form(self, geometry: int, form: int, blocks_per_cu: int, stream: int = 0, store: int = L.STORE_AUTO):
        """One row tile per block in kernel form ``form`` (skipln_tune_forward_form)."""
        w = self.w
        p = lambda t: None if t is None else t.data_ptr()
        st = L.load_tune().skipln_tune_forward_form(
            OPS[w.op], p(self.x), p(self.skip), skip_mode(w), w.skip_rows if w.broadcast else 0, p(self.gamma),
            p(self.beta), p(self.bias), p(self.out), p(self.res), w.rows, w.hidden, float(np.float32(w.eps)),
            L.F32 if w.dtype == "f32" else L.F16, geometry, form, blocks_per_cu, store, stream or None)
        L.check(st, "skipln_tune_forward_form")

    def host(self, t):
        import torch

        torch.cuda.synchronize()
        return t.cpu().numpy().reshape(self.w.rows, self.w.hidden)


def oracle_rows(w, inputs, row_offset: int = 0, threads: int = 8):
    """The oracle's result for ``w.op``: {"y": binary64 output, "residual": T}
    for the normalizations and BiasSoftmax; {"y": Y in T (BiasAdd's output is
    exact)}.  ``inputs["input"]`` may hold rows ``row_offset ..`` only."""
    if w.op == "bias_softmax":
        n = inputs["input"].shape[0]
        if row_offset == 0 and n == w.rows:
            y = O.bias_softmax(inputs["input"], inputs["skip"], w.inner)
        else:
            # A slice of rows: hand the oracle the bias row each one reads.
            bias = inputs["skip"][w.skip_row_of(np.arange(row_offset, row_offset + n))]
            y = O.bias_softmax(inputs["input"], bias, False)
        return {"y": y, "residual": None}
    if w.op == "bias_add":
        y, _ = O.bias_add(inputs["input"], inputs["bias"], inputs["skip"])
        return {"y": y, "residual": None}
    return O.skip_layer_norm(inputs["input"], inputs["skip"], inputs["gamma"], inputs["beta"], inputs["bias"],
                             w.eps, broadcast=w.broadcast, row_offset=row_offset, residual=True, threads=threads,
                             simplified=w.op == "simplified")


def compare(w, got_out, got_res, ref):
    """BiasAdd: output bit for bit.  Normalizations: output within tolerance
    of the binary64 value, residual bit for bit when emitted."""
    if w.op == "bias_add":
        assert_bits_equal(got_out, ref["y"], "bias_add output")
        return
    if w.op == "bias_softmax":
        assert_out_close(got_out, ref["y"], w.dtype, "softmax out", tol=SOFTMAX_TOL)
        return
    assert_out_close(got_out, ref["y"], w.dtype)
    if got_res is not None:
        assert_bits_equal(got_res, ref["residual"])


def assert_out_close(got: np.ndarray, want: np.ndarray, dt: str, what: str = "out", tol=None):
    atol, rtol = (TOL if tol is None else tol)[dt]
    g = got.astype(np.float64)
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(g), nan_w), f"{what}: NaN pattern differs ({int(np.isnan(g).sum())} vs " \
                                               f"{int(nan_w.sum())})"
    err = np.abs(g[~nan_w] - want[~nan_w])
    lim = atol + rtol * np.abs(want[~nan_w])
    bad = err > lim
    if bad.any():
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside {atol}+{rtol}|y|; "
                             f"worst err {err[i]:.3e} at y={want[~nan_w][i]:.6g}")


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str = "residual"):
    gb = np.ascontiguousarray(got).view(np.uint16 if got.dtype == np.float16 else np.uint32)
    wb = np.ascontiguousarray(want).view(np.uint16 if want.dtype == np.float16 else np.uint32)
    if not np.array_equal(gb, wb):
        diff = gb != wb
        idx = np.argwhere(diff)[0]
        raise AssertionError(f"{what}: {int(diff.sum())} elements differ bitwise; first at {tuple(idx)}: "
                             f"{got[tuple(idx)]!r} vs {want[tuple(idx)]!r}")


def check_case(w, variant: int = L.VARIANT_AUTO, offset_elems: int = 0, inputs=None, workspace=None):
    """Run one workload through the C ABI and compare all rows with the oracle."""
    from transformer_residual_add_amd import workloads as W

    inputs = W.make_inputs(w) if inputs is None else inputs
    dc = DeviceCase(w, inputs, residual=w.residual, offset_elems=offset_elems)
    dc.run(variant, workspace=workspace)
    ref = oracle_rows(w, inputs)
    compare(w, dc.host(dc.out), dc.host(dc.res) if w.residual else None, ref)
    return dc, ref
