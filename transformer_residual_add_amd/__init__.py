"""MI355X-native SkipLayerNormalization (com.microsoft contrib operator).

``skip_layer_norm`` computes, row by row over the hidden axis,
``s = input + skip (+ bias)`` and ``(s - mean) / sqrt(var + epsilon) * gamma
(+ beta)``, optionally returning ``s`` as ``input_skip_bias_sum``
(com.microsoft SkipLayerNormalization WebGPU manifest: `description`,
`inputs`, `outputs`, `attributes.epsilon`).  ``bias_add`` and
``bias_softmax`` are the com.microsoft BiasAdd and BiasSoftmax operators on the
same row kernels.  The computation runs in the HIP kernels of
``libskipln.so``; PyTorch only provides device memory and streams.
"""
from __future__ import annotations

from typing import Optional

from . import _lib
from ._lib import SkiplnArgumentError, SkiplnError  # noqa: F401

# The manifest's default epsilon: 1e-12 rounded to binary32
# (SkipLayerNormalization manifest, `attributes.epsilon`).
DEFAULT_EPSILON = 9.999999960041972e-13

__all__ = ["skip_layer_norm", "bias_add", "bias_softmax", "bias_softmax_raw", "softmax_shape", "forward_raw",
           "workspace_bytes", "select_kernel", "SkiplnError", "SkiplnArgumentError", "DEFAULT_EPSILON"]


def forward_raw(input_ptr: int, skip_ptr: int, skip_mode: int, skip_rows: int, gamma_ptr: Optional[int],
                beta_ptr: Optional[int], bias_ptr: Optional[int], out_ptr: int, residual_ptr: Optional[int],
                rows: int, hidden: int, eps: float, dtype: int, stream: int = 0,
                variant: int = _lib.VARIANT_AUTO, op: int = _lib.OP_LAYER_NORM,
                workspace: Optional[tuple] = None) -> None:
    """Operation ``op`` on raw device pointers; raises SkiplnError.

    The automatic kernel choice goes through the operator library: the
    operation's own entry point, or ``skipln_forward_ws`` when ``workspace`` =
    (pointer, bytes) is given.  A forced kernel family (``variant``) goes
    through the tuning library's ``skipln_tune_forward``."""
    ws_ptr, ws_bytes = workspace if workspace is not None else (None, 0)
    args = (input_ptr, skip_ptr, skip_mode, skip_rows, gamma_ptr or None, beta_ptr or None, bias_ptr or None,
            out_ptr, residual_ptr or None, rows, hidden, eps, dtype)
    if variant != _lib.VARIANT_AUTO:
        st = _lib.load_tune().skipln_tune_forward(op, *args, variant, ws_ptr or None, ws_bytes, stream or None)
        _lib.check(st, "skipln_tune_forward")
        return
    lib = _lib.load()
    if workspace is not None:
        st = lib.skipln_forward_ws(op, *args, ws_ptr or None, ws_bytes, stream or None)
    elif op == _lib.OP_LAYER_NORM:
        st = lib.skipln_forward(*args, stream or None)
    elif op == _lib.OP_SIMPLIFIED:
        st = lib.skipln_forward_simplified(*args, stream or None)
    elif op == _lib.OP_BIAS_ADD:
        if skip_mode != _lib.SKIP_EXACT:
            _lib.check(_lib.ERR_MODE, "skipln_bias_add")
        st = lib.skipln_bias_add(input_ptr, bias_ptr or None, skip_ptr, out_ptr, rows, hidden, dtype, stream or None)
    elif op == _lib.OP_BIAS_SOFTMAX:
        bias_rows = rows if skip_mode == _lib.SKIP_EXACT else skip_rows
        st = lib.skipln_bias_softmax(input_ptr, skip_ptr, out_ptr, rows, hidden, bias_rows,
                                     1 if skip_mode == _lib.SKIP_BROADCAST_INNER else 0, dtype, None, 0,
                                     stream or None)
    else:
        _lib.check(_lib.ERR_OP, "forward_raw")
    _lib.check(st, "skipln_forward")


def workspace_bytes(op: int, rows: int, hidden: int, dtype: int, skip_mode: int = _lib.SKIP_EXACT,
                    skip_rows: int = 0, variant: int = _lib.VARIANT_AUTO) -> int:
    """Device workspace a call with these arguments may need (0: none): the
    operator library's ``skipln_workspace_bytes`` for the automatic choice,
    the tuning library's for a forced kernel family."""
    if variant == _lib.VARIANT_AUTO:
        n = _lib.load().skipln_workspace_bytes(op, rows, hidden, dtype, skip_mode, skip_rows)
    else:
        n = _lib.load_tune().skipln_tune_workspace_bytes(op, rows, hidden, dtype, skip_mode, skip_rows, variant)
    if n < 0:
        _lib.check(-n, "skipln_workspace_bytes")
    return int(n)


def _hold(t, stream) -> None:
    """Keep workspace ``t`` (allocated on the current stream) from being reused
    before work enqueued on ``stream`` ends."""
    import torch

    if t is None or stream is None:
        return
    t.record_stream(torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream)


def _workspace(nbytes: int, device):
    """(tensor, (pointer, bytes)) of a device workspace, or (None, None)."""
    import torch

    if nbytes <= 0:
        return None, None
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t, (t.data_ptr(), nbytes)


def bias_softmax_raw(data_ptr: int, bias_ptr: int, out_ptr: int, batch_count: int, block_size: int,
                     bias_batch_count: int, is_inner_broadcast: bool, dtype: int, stream: int = 0,
                     workspace: Optional[tuple] = None) -> None:
    """``skipln_bias_softmax`` on raw device pointers (``workspace`` = (pointer,
    bytes) or None); raises SkiplnError."""
    ws_ptr, ws_bytes = workspace if workspace is not None else (None, 0)
    st = _lib.load().skipln_bias_softmax(data_ptr or None, bias_ptr or None, out_ptr or None, batch_count,
                                         block_size, bias_batch_count, 1 if is_inner_broadcast else 0, dtype,
                                         ws_ptr or None, ws_bytes, stream or None)
    _lib.check(st, "skipln_bias_softmax")


def select_kernel(hidden: int, dtype: int, aligned16: bool = True, variant: int = _lib.VARIANT_AUTO,
                  skip_mode: int = _lib.SKIP_EXACT, op: int = _lib.OP_LAYER_NORM, workspace: bool = False,
                  rows: int = -1, cus: int = 0) -> str:
    """Name of the kernel a call with this operation, row count (-1: fewer than
    the device's compute units), hidden size and skip form would launch
    (``workspace``: a call that brings one; ``cus`` <= 0: the current
    device's compute units)."""
    kid = _lib.load_tune().skipln_tune_select(op, rows, hidden, dtype, skip_mode, 1 if aligned16 else 0, variant,
                                              1 if workspace else 0, cus)
    if kid < 0:
        _lib.check(-kid, "skipln_tune_select")
    return _lib.kernel_name(kid)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return _lib.F32
    if t.dtype == torch.float16:
        return _lib.F16
    raise TypeError(f"SkipLayerNormalization supports float32 and float16, got {t.dtype}")


def _check_tensors(input, tensors):
    for t in tensors:
        if t.dtype != input.dtype:
            raise TypeError("all tensors must share one dtype")
        if t.device != input.device or t.device.type != "cuda":
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream if isinstance(stream, int) else stream.cuda_stream


def skip_layer_norm(input, skip, gamma, beta=None, bias=None, epsilon: float = DEFAULT_EPSILON, *,
                    return_residual: bool = False, out=None, residual_out=None, stream=None,
                    variant: int = _lib.VARIANT_AUTO, simplified: bool = False):
    """SkipLayerNormalization on CUDA (HIP) tensors.

    input: (N, S, H) or (rows, H).  skip: the input's shape, or for rank-3
    input (1, S, H) or (S, H), broadcast over the batch.  gamma (H), optional
    beta (H) and bias (H).  All tensors contiguous, of one dtype (float32 or
    float16), on one device.  Returns ``out``, or ``(out, residual)`` with
    ``return_residual=True`` (the input_skip_bias_sum output).
    ``simplified=True`` selects the root-mean-square form (no mean
    subtraction, mean square in place of the variance).
    """
    import torch

    tensors = [t for t in (input, skip, gamma, beta, bias, out, residual_out) if t is not None]
    code = _dtype_code(input)
    _check_tensors(input, tensors)
    if input.dim() not in (2, 3):
        raise ValueError("input must have rank 2 or 3")
    h = input.shape[-1]
    rows = input.numel() // h if h else 0
    if tuple(skip.shape) == tuple(input.shape):
        mode, skip_rows = _lib.SKIP_EXACT, 0
    elif input.dim() == 3 and tuple(skip.shape) in ((1,) + tuple(input.shape[1:]), tuple(input.shape[1:])):
        mode, skip_rows = _lib.SKIP_BROADCAST, input.shape[1]
    else:
        raise ValueError(f"skip shape {tuple(skip.shape)} does not fit input {tuple(input.shape)}")
    for name, t in (("gamma", gamma), ("beta", beta), ("bias", bias)):
        if t is not None and tuple(t.shape) != (h,):
            raise ValueError(f"{name} must have shape ({h},)")
    if out is None:
        out = torch.empty_like(input)
    elif out.shape != input.shape:
        raise ValueError("out must have the input's shape")
    if return_residual and residual_out is None:
        residual_out = torch.empty_like(input)
    if residual_out is not None and residual_out.shape != input.shape:
        raise ValueError("residual_out must have the input's shape")
    s = _stream_handle(stream, input.device)
    op = _lib.OP_SIMPLIFIED if simplified else _lib.OP_LAYER_NORM
    with torch.cuda.device(input.device):
        # Rows too long for one workgroup split across workgroups through a
        # small workspace (torch's caching allocator provides it).
        ws_t, ws = _workspace(workspace_bytes(op, rows, h, code, mode, skip_rows, variant) if rows else 0,
                              input.device)
        forward_raw(input.data_ptr(), skip.data_ptr(), mode, skip_rows, gamma.data_ptr(),
                    beta.data_ptr() if beta is not None else None,
                    bias.data_ptr() if bias is not None else None, out.data_ptr(),
                    residual_out.data_ptr() if residual_out is not None else None,
                    rows, h, float(epsilon), code, s, variant, op, workspace=ws)
        _hold(ws_t, stream)
    if return_residual:
        return out, residual_out
    return out


def bias_add(X, bias, skip, *, out=None, stream=None, variant: int = _lib.VARIANT_AUTO):
    """BiasAdd on CUDA (HIP) tensors: ``(X + bias) + skip``.

    X and skip: (N, S, C) (or any shape whose last axis is C), bias: (C,).
    All tensors contiguous, of one dtype (float32 or float16), on one device.
    """
    import torch

    code = _dtype_code(X)
    _check_tensors(X, [t for t in (X, bias, skip, out) if t is not None])
    if X.dim() < 1 or tuple(skip.shape) != tuple(X.shape):
        raise ValueError("skip must have X's shape")
    c = X.shape[-1]
    if tuple(bias.shape) != (c,):
        raise ValueError(f"bias must have shape ({c},)")
    if out is None:
        out = torch.empty_like(X)
    elif out.shape != X.shape:
        raise ValueError("out must have X's shape")
    rows = X.numel() // c if c else 0
    s = _stream_handle(stream, X.device)
    with torch.cuda.device(X.device):
        forward_raw(X.data_ptr(), skip.data_ptr(), _lib.SKIP_EXACT, 0, None, None, bias.data_ptr(), out.data_ptr(),
                    None, rows, c, 0.0, code, s, variant, _lib.OP_BIAS_ADD)
    return out


def softmax_shape(data_shape, bias_numel: int, axis: int = 1):
    """(batch_count, block_size, bias_batch_count) of BiasSoftmax for a data
    shape, a bias element count and ``axis`` (BiasSoftmax manifest,
    `derive.axisNorm`, `batchCount`, `blockSize`, `biasBlockCount`)."""
    rank = len(data_shape)
    if rank < 1 or not -rank <= axis < rank:
        raise ValueError(f"axis {axis} out of range for rank {rank}")
    a = axis if axis >= 0 else axis + rank
    batch = 1
    for d in data_shape[:a]:
        batch *= int(d)
    block = 1
    for d in data_shape[a:]:
        block *= int(d)
    if block > 0 and bias_numel % block != 0:
        raise ValueError(f"bias has {bias_numel} elements, not a whole number of rows of {block}")
    return batch, block, (bias_numel // block if block > 0 else 0)


def bias_softmax(data, bias, is_inner_broadcast: bool, axis: int = 1, *, out=None, stream=None,
                 variant: int = _lib.VARIANT_AUTO):
    """BiasSoftmax on CUDA (HIP) tensors: ``softmax(data + bias)`` over the
    flattened dimensions from ``axis`` on.

    The bias holds a whole number of softmax rows, a divisor of the data's row
    count; they are reused by consecutive groups of rows
    (``is_inner_broadcast=True``) or cyclically (False).  Tensors contiguous,
    of one dtype (float32 or float16), on one device.
    """
    import torch

    code = _dtype_code(data)
    _check_tensors(data, [t for t in (data, bias, out) if t is not None])
    batch, block, bias_rows = softmax_shape(tuple(data.shape), bias.numel(), axis)
    if out is None:
        out = torch.empty_like(data)
    elif out.shape != data.shape:
        raise ValueError("out must have data's shape")
    s = _stream_handle(stream, data.device)
    mode = (_lib.SKIP_EXACT if bias_rows == batch
            else _lib.SKIP_BROADCAST_INNER if is_inner_broadcast else _lib.SKIP_BROADCAST)
    with torch.cuda.device(data.device):
        ws_t, ws = None, None
        if batch * block > 0 and 0 < bias_rows <= batch and batch % bias_rows == 0:
            ws_t, ws = _workspace(workspace_bytes(_lib.OP_BIAS_SOFTMAX, batch, block, code, mode, bias_rows, variant),
                                  data.device)
        if variant == _lib.VARIANT_AUTO:
            bias_softmax_raw(data.data_ptr(), bias.data_ptr(), out.data_ptr(), batch, block, bias_rows,
                             is_inner_broadcast, code, s, workspace=ws)
        elif batch * block > 0:
            forward_raw(data.data_ptr(), bias.data_ptr(), mode, bias_rows, None, None, None, out.data_ptr(), None,
                        batch, block, 0.0, code, s, variant, _lib.OP_BIAS_SOFTMAX, workspace=ws)
        _hold(ws_t, stream)
    return out
