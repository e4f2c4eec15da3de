"""GPU parity on both sides of every switch point of the automatic kernel
choice.

The switch points are read from the library itself at collection time: for
each operation, element type and skip form, the row length is scanned (in
whole 16-byte chunks, and separately over lengths that are not whole
chunks) and wherever the kernel that `skipln_tune_select` names changes,
the last length of the old kernel and the first of the new one are both
run through the operator and compared with the oracle over every row.  Rows
past one workgroup's LDS are also run with a workspace (the split-row
kernels) where the choice takes them.  The tolerances are those of the other
parity tests (gpu_util).
"""
import pytest

import transformer_residual_add_amd as T
from transformer_residual_add_amd import _lib as L
from transformer_residual_add_amd import workloads as W

import gpu_util as U

pytestmark = pytest.mark.gpu

CUS = 256  # the choice is scanned for a 256-CU device; rows below are fewer
OPS = [("layer_norm", L.OP_LAYER_NORM), ("simplified", L.OP_SIMPLIFIED), ("bias_add", L.OP_BIAS_ADD),
       ("bias_softmax", L.OP_BIAS_SOFTMAX)]


def _rows(hidden: int) -> int:
    return 19 if hidden <= 8192 else 3


def _switch_points(op: int, dtype: int, mode: int, ragged: bool, workspace: bool):
    """Row lengths on either side of each change of the chosen kernel."""
    tune = L.load_tune()
    v = 4 if dtype == L.F32 else 8
    if ragged:
        lengths = [h for h in range(1, 16400) if h % v]
    else:
        top = 163840 + 2 * v if op == L.OP_BIAS_SOFTMAX else 45056
        lengths = list(range(v, top + 1, v))
    points = set()
    prev = None
    for h in lengths:
        k = tune.skipln_tune_select(op, _rows(h), h, dtype, mode, 1, L.VARIANT_AUTO, 1 if workspace else 0, CUS)
        if prev is not None and k != prev[1]:
            points.add(prev[0])
            points.add(h)
        prev = (h, k)
    return sorted(points)


def _cases():
    out = []
    for name, op in OPS:
        for dt, code in (("f32", L.F32), ("f16", L.F16)):
            modes = [L.SKIP_EXACT, L.SKIP_BROADCAST] if op in (L.OP_LAYER_NORM, L.OP_SIMPLIFIED) else [L.SKIP_EXACT]
            for mode in modes:
                form = "bcast" if mode == L.SKIP_BROADCAST else "exact"
                for ragged in (False, True):
                    for h in _switch_points(op, code, mode, ragged, False):
                        out.append(pytest.param(name, dt, mode, h, False, id=f"{name}-{dt}-{form}-{h}"))
                # With a workspace the longest rows may take the split-row kernels.
                for h in _switch_points(op, code, mode, False, True):
                    if h > 40000:
                        out.append(pytest.param(name, dt, mode, h, True, id=f"{name}-{dt}-{form}-{h}-ws"))
    return out


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("op,dt,mode,hidden,with_ws", _cases())
def test_both_sides_of_each_switch(op, dt, mode, hidden, with_ws):
    rows = _rows(hidden)
    bcast = mode == L.SKIP_BROADCAST
    if bcast:
        rows = 18 if hidden <= 8192 else 4
    softmax = op == "bias_softmax"
    w = W.small_case(rows, hidden, dt, skip_rows=(rows // 3 if hidden <= 8192 else 2) if bcast else None,
                     beta=True, bias=not softmax, residual=True, eps=1e-5, seed=hidden * 7 + (3 if bcast else 0),
                     op=op)
    code = L.F32 if dt == "f32" else L.F16
    inputs = W.make_inputs(w)
    ws = None
    if with_ws:
        n = T.workspace_bytes(U.OPS[op], w.rows, w.hidden, code, U.skip_mode(w), w.skip_rows if w.broadcast else 0)
        if n > 0:
            import torch

            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    kernel = T.select_kernel(hidden, code, True, L.VARIANT_AUTO, U.skip_mode(w), U.OPS[op], workspace=ws is not None,
                             rows=w.rows)
    U.note(f"switch {op} {dt} {'bcast' if bcast else 'exact'} rows={w.rows} H={hidden} ws={ws is not None} "
           f"kernel={kernel}")
    U.check_case(w, inputs=inputs, workspace=None if ws is None else (ws.data_ptr(), ws.numel()))
