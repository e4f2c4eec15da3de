"""skipln_forward_ws_static (no allocation, library-held scratch) against
skipln_forward_ws (caller workspace) through the C ABI: the same kernels on
the same inputs give the same bits, call after call, the second call of each
pair smaller than the first; both also within tolerance of the oracle.  And
the call such callers make it for: captured in a HIP graph and replayed."""
import numpy as np
import pytest

from transformer_residual_add_amd import _lib as L
from transformer_residual_add_amd import workloads as W

import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L.load()
    yield
    torch.cuda.synchronize()


def _call(entry, w, dc, out, res, ws=None, stream=None):
    p = lambda t: None if t is None else t.data_ptr()
    args = (U.OPS[w.op], p(dc.x), p(dc.skip), U.skip_mode(w), w.skip_rows if w.broadcast else 0, p(dc.gamma),
            p(dc.beta), p(dc.bias), p(out), p(res), w.rows, w.hidden, float(np.float32(w.eps)),
            L.F32 if w.dtype == "f32" else L.F16)
    lib = L.load()
    if entry == "static":
        st = lib.skipln_forward_ws_static(*args, stream)
    else:
        st = lib.skipln_forward_ws(*args, ws[0], ws[1], stream)
    L.check(st, f"skipln_forward_ws{'_static' if entry == 'static' else ''}")


def _case(rows, hidden, dt, op, seed, skip_rows=None):
    return W.small_case(rows, hidden, dt, skip_rows=skip_rows, beta=op != "bias_softmax", bias=op != "bias_softmax",
                        residual=op != "bias_softmax", eps=1e-5, seed=seed, op=op)


PAIRS = [
    ("layer_norm_f32", _case(16, 100000, "f32", "layer_norm", 1), _case(5, 70000, "f32", "layer_norm", 2)),
    ("simplified_f16", _case(12, 131072, "f16", "simplified", 3), _case(3, 49152, "f16", "simplified", 4)),
    ("layer_norm_f16_bcast", _case(8, 131072, "f16", "layer_norm", 5, skip_rows=2),
     _case(2, 81920, "f16", "layer_norm", 6)),
    ("softmax_f32", _case(4, 100000, "f32", "bias_softmax", 7), _case(2, 90000, "f32", "bias_softmax", 8)),
    ("layer_norm_f32_no_split", _case(64, 1024, "f32", "layer_norm", 9), _case(7, 768, "f32", "layer_norm", 10)),
]


@pytest.mark.parametrize("name,big,small", PAIRS, ids=[p[0] for p in PAIRS])
def test_static_scratch_matches_caller_workspace(name, big, small):
    import torch

    cases = []
    for w in (big, small):
        inputs = W.make_inputs(w)
        dc = U.DeviceCase(w, inputs, residual=w.residual)
        dt = U.torch_dtype(w.dtype)
        n = w.rows * w.hidden
        ref_out = torch.full((n,), float("nan"), dtype=dt, device="cuda")
        ref_res = torch.full((n,), float("nan"), dtype=dt, device="cuda") if w.residual else None
        cases.append((w, inputs, dc, ref_out, ref_res))
    # The existing entry point with a caller workspace, as reference.
    for w, inputs, dc, ref_out, ref_res in cases:
        ws = dc.workspace()
        U.note(f"no-alloc {name}: skipln_forward_ws rows={w.rows} H={w.hidden} workspace={ws[1]}")
        _call("ws", w, dc, ref_out, ref_res, ws=ws if ws[1] > 0 else (None, 0))
    # Two calls in a row through the static scratch, the second smaller.
    for w, inputs, dc, ref_out, ref_res in cases:
        U.note(f"no-alloc {name}: skipln_forward_ws_static rows={w.rows} H={w.hidden}")
        _call("static", w, dc, dc.out, dc.res)
    torch.cuda.synchronize()
    for w, inputs, dc, ref_out, ref_res in cases:
        got, want = dc.host(dc.out), ref_out.cpu().numpy().reshape(w.rows, w.hidden)
        U.assert_bits_equal(got, want, f"{name} out rows={w.rows}")
        if w.residual:
            U.assert_bits_equal(dc.host(dc.res), ref_res.cpu().numpy().reshape(w.rows, w.hidden),
                                f"{name} residual rows={w.rows}")
        U.compare(w, got, dc.host(dc.res) if w.residual else None, U.oracle_rows(w, inputs))


def test_static_scratch_under_graph_capture():
    """A split-row layer norm through skipln_forward_ws_static, captured in a
    HIP graph on a side stream and replayed three times; between replays an
    eager call of another shape goes through the same scratch.  Every replay
    writes the eager call's bits (the kernels clear nothing with memsets, so
    the graph holds kernel nodes only)."""
    import torch

    big, other = _case(16, 100000, "f32", "layer_norm", 11), _case(5, 70000, "f32", "layer_norm", 12)
    dcs = {}
    for w in (big, other):
        dcs[w.name] = U.DeviceCase(w, W.make_inputs(w), residual=True)
    dc, dco = dcs[big.name], dcs[other.name]
    U.note(f"no-alloc graph: eager rows={big.rows} H={big.hidden}")
    _call("static", big, dc, dc.out, dc.res)
    torch.cuda.synchronize()
    want_out, want_res = dc.out.clone(), dc.res.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _call("static", big, dc, dc.out, dc.res, stream=s.cuda_stream)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    U.note("no-alloc graph: capture")
    with torch.cuda.graph(g, stream=s):
        _call("static", big, dc, dc.out, dc.res, stream=s.cuda_stream)
    for i in range(3):
        U.note(f"no-alloc graph: eager call rows={other.rows} H={other.hidden}, then replay {i}")
        _call("static", other, dco, dco.out, dco.res)
        dc.out.fill_(float("nan"))
        dc.res.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc.out.view(torch.int32), want_out.view(torch.int32)), f"replay {i}: output bits"
        assert torch.equal(dc.res.view(torch.int32), want_res.view(torch.int32)), f"replay {i}: residual bits"
    inputs = W.make_inputs(big)
    U.compare(big, dc.host(dc.out), dc.host(dc.res), U.oracle_rows(big, inputs))
