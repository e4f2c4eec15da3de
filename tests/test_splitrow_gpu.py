"""GPU parity of the split-row kernels: rows cut into 16 KiB slices, one
workgroup per slice, partial results merged through a workspace -- layer
normalization, its root-mean-square form and BiasSoftmax, against the
oracle with the same tolerances as the single-workgroup kernels."""
import numpy as np
import pytest

import transformer_residual_add_amd as T
from transformer_residual_add_amd import _lib as L
from transformer_residual_add_amd import workloads as W

import gpu_util as U

pytestmark = pytest.mark.gpu

SPLIT = L.VARIANT_SPLITROW


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L.load()
    yield
    torch.cuda.synchronize()


def norm_case(rows, hidden, dt, op, bcast=False, flags=(True, True, True), seed=1, mu=0.0):
    beta, bias, residual = flags
    return W.small_case(rows, hidden, dt, skip_rows=4 if bcast else None, beta=beta, bias=bias, residual=residual,
                        eps=1e-5, seed=seed, input_dist=W.normal(mu, 1), op=op)


def softmax_case(rows, hidden, dt, mode="exact", seed=1, bias_rows=4):
    return W.small_case(rows, hidden, dt, skip_rows=None if mode == "exact" else bias_rows, seed=seed,
                        input_dist=W.normal(0, 2), skip_dist=W.normal(0, 1), op="bias_softmax",
                        inner=mode == "inner")


# one slice (ragged and full), several slices with a ragged last one, many slices
SIZES_F32 = [4, 64, 4096, 4100, 12288, 40960, 65536, 100000]
SIZES_F16 = [8, 64, 8192, 8200, 40960, 131072, 128256]


@pytest.mark.parametrize("op", ["layer_norm", "simplified"])
@pytest.mark.parametrize("dt_hidden", [("f32", h) for h in SIZES_F32] + [("f16", h) for h in SIZES_F16],
                         ids=lambda t: f"{t[0]}_h{t[1]}")
@pytest.mark.parametrize("form", [(False, (True, True, True)), (True, (False, False, False)),
                                  (False, (True, False, True))], ids=["exact_all", "bcast_none", "exact_beta_res"])
def test_split_normalizations(op, dt_hidden, form):
    dt, hidden = dt_hidden
    bcast, flags = form
    rows = 12 if hidden > 50000 else 24
    w = norm_case(rows, hidden, dt, op, bcast, flags, seed=hidden % 977)
    U.note(f"split {op} {dt} H={hidden} bcast={bcast} flags={flags}")
    U.check_case(w, variant=SPLIT, workspace=True)


@pytest.mark.parametrize("dt_hidden", [("f32", h) for h in SIZES_F32] + [("f16", h) for h in SIZES_F16],
                         ids=lambda t: f"{t[0]}_h{t[1]}")
@pytest.mark.parametrize("mode", ["exact", "outer", "inner"])
def test_split_softmax(dt_hidden, mode):
    dt, hidden = dt_hidden
    rows = 12 if hidden > 50000 else 24
    w = softmax_case(rows, hidden, dt, mode, seed=hidden % 991)
    U.note(f"split softmax {dt} H={hidden} {mode}")
    U.check_case(w, variant=SPLIT, workspace=True)


@pytest.mark.parametrize("dt,hidden,op", [("f32", 100000, "layer_norm"), ("f16", 131072, "simplified"),
                                          ("f32", 98304, "bias_softmax"), ("f16", 163848, "bias_softmax"),
                                          ("f32", 262144, "layer_norm")])
def test_split_auto_with_workspace(dt, hidden, op):
    """Rows beyond the LDS capacity and beyond the registers of one block:
    the automatic choice with a workspace."""
    code = L.F32 if dt == "f32" else L.F16
    assert T.select_kernel(hidden, code, op=U.OPS[op], workspace=True).endswith(f"splitrow_{dt}")
    w = (softmax_case(8, hidden, dt, "inner", bias_rows=2) if op == "bias_softmax"
         else norm_case(8, hidden, dt, op, seed=3))
    U.note(f"split auto {op} {dt} H={hidden}")
    U.check_case(w, workspace=True)


@pytest.mark.parametrize("dt,hidden", [("f32", 65536), ("f16", 131072)])
def test_split_many_rows(dt, hidden):
    """More rows than one batch holds (128 MiB of streamed inputs): the
    workspace is reused batch after batch on the same stream."""
    rows = 519
    w = norm_case(rows, hidden, dt, "layer_norm", seed=11)
    U.note(f"split many rows {dt} H={hidden} rows={rows}")
    U.check_case(w, variant=SPLIT, workspace=True)


@pytest.mark.parametrize("dt,hidden,op", [("f16", 131072, "simplified"), ("f32", 262144, "simplified")])
def test_many_rows_auto_takes_generic(dt, hidden, op):
    """With a row for every CU, RMS rows beyond the registers' 65536 values
    take the generic kernel even when a workspace is at hand (with fewer
    rows, the split-row pair): the kernel
    choice for the call's row count on this device says so, and the call
    through skipln_forward_ws (with the workspace the size query asks for,
    unused) and through the allocating wrapper match the oracle."""
    import torch

    rows = torch.cuda.get_device_properties(0).multi_processor_count  # a row for every CU
    w = norm_case(rows, hidden, dt, op, seed=13, mu=100.0 if op == "layer_norm" else 0.0)
    code = L.F32 if dt == "f32" else L.F16
    assert T.select_kernel(hidden, code, op=U.OPS[op], workspace=True, rows=rows).split("_")[-2] == "generic"
    assert T.select_kernel(hidden, code, op=U.OPS[op], workspace=True, rows=rows - 1).split("_")[-2] == "splitrow"
    inputs = W.make_inputs(w)
    ref = U.oracle_rows(w, inputs)
    U.note(f"auto many rows {op} {dt} H={hidden} rows={rows}")
    dc = U.DeviceCase(w, inputs, residual=True)
    dc.run(L.VARIANT_AUTO, workspace=True)
    U.compare(w, dc.host(dc.out), dc.host(dc.res), ref)
    tt = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out, res = T.skip_layer_norm(tt(inputs["input"]), tt(inputs["skip"]), tt(inputs["gamma"]), tt(inputs["beta"]),
                                 tt(inputs["bias"]), epsilon=float(w.eps), return_residual=True,
                                 simplified=op == "simplified")
    torch.cuda.synchronize()
    U.compare(w, out.cpu().numpy().reshape(rows, hidden), res.cpu().numpy().reshape(rows, hidden), ref)


def test_split_workspace_errors_enqueue_nothing():
    import torch

    w = norm_case(4, 100000, "f32", "layer_norm", seed=2)
    dc = U.DeviceCase(w, W.make_inputs(w), residual=True)
    ptr, need = dc.workspace()
    before = dc.out.clone()
    for ws in ((None, 0), (ptr, need - 16), (ptr + 8, need)):
        with pytest.raises(T.SkiplnError) as e:
            dc.run(workspace=ws)
        assert e.value.status == L.ERR_WORKSPACE
    with pytest.raises(T.SkiplnError) as e:
        dc.run(workspace=(dc.x.data_ptr(), need))
    assert e.value.status == L.ERR_ALIAS
    torch.cuda.synchronize()
    assert torch.equal(dc.out.view(torch.int32), before.view(torch.int32))


def test_split_wrappers_allocate_their_workspace():
    import torch

    from oracle import oracle as O

    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 3, 65536)).astype(np.float32)
    sk = rng.standard_normal((2, 3, 65536)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 65536).astype(np.float32)
    out, res = T.skip_layer_norm(torch.from_numpy(x).cuda(), torch.from_numpy(sk).cuda(), torch.from_numpy(g).cuda(),
                                 epsilon=1e-5, return_residual=True)
    torch.cuda.synchronize()
    ref = O.skip_layer_norm(x.reshape(6, -1), sk.reshape(6, -1), g, None, None, 1e-5, residual=True)
    U.assert_out_close(out.cpu().numpy().reshape(6, -1), ref["y"], "f32")
    U.assert_bits_equal(res.cpu().numpy().reshape(6, -1), ref["residual"])
    logits = (rng.standard_normal((4, 1, 128256)) * 3).astype(np.float16)
    bias = (rng.standard_normal(128256)).astype(np.float16)
    y = T.bias_softmax(torch.from_numpy(logits).cuda(), torch.from_numpy(bias).cuda(), True, axis=-1)
    torch.cuda.synchronize()
    ref = O.bias_softmax(logits.reshape(4, -1), bias.reshape(1, -1), True)
    U.assert_out_close(y.cpu().numpy().reshape(4, -1), ref, "f16", "vocab softmax", tol=U.SOFTMAX_TOL)
    # on a side stream: the workspace outlives the call until the stream's work ends
    s = torch.cuda.Stream()
    ld, bd = torch.from_numpy(logits).cuda(), torch.from_numpy(bias).cuda()
    s.wait_stream(torch.cuda.current_stream())
    y2 = T.bias_softmax(ld, bd, True, axis=-1, stream=s)
    s.synchronize()
    assert torch.equal(y2, y)


def test_split_graph_replay():
    import torch

    w = softmax_case(16, 65536, "f32", "outer", bias_rows=4, seed=5)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=False)
    ws = dc.workspace()
    dc.run(workspace=ws)
    first = dc.out.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dc.run(stream=s.cuda_stream, workspace=ws)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dc.run(stream=s.cuda_stream, workspace=ws)
    for _ in range(3):
        dc.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc.out.view(torch.int32), first.view(torch.int32))
    U.compare(w, dc.host(dc.out), None, U.oracle_rows(w, inputs))


@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_softmax"])
@pytest.mark.parametrize("over", ["input", "skip"])
def test_split_in_place(op, over):
    """out over the input (or the exact skip): a workgroup reads its own
    slice before writing it.  A residual over an input cannot take the
    split-row kernels: forced, the call is refused; automatic, it runs the
    generic kernel."""
    dt, hidden = "f32", 65536
    w = (softmax_case(16, hidden, dt, "exact", seed=7) if op == "bias_softmax"
         else norm_case(16, hidden, dt, op, seed=7, mu=100.0))
    inputs = W.make_inputs(w)
    ref = U.oracle_rows(w, inputs)
    norm = op != "bias_softmax"
    dc = U.DeviceCase(w, inputs, residual=norm)
    U.note(f"split in place {op} over {over}")
    target = dc.x if over == "input" else dc.skip
    dc.run(SPLIT, out=target, workspace=dc.workspace(SPLIT))
    U.compare(w, dc.host(target), dc.host(dc.res) if norm else None, ref)
    if norm:
        dc2 = U.DeviceCase(w, inputs, residual=True)
        other = dc2.skip if over == "input" else dc2.x
        with pytest.raises(T.SkiplnError) as e:
            dc2.run(SPLIT, out=dc2.out, res=other, workspace=dc2.workspace(SPLIT))
        assert e.value.status == L.ERR_UNSUPPORTED
        dc2.run(L.VARIANT_AUTO, out=dc2.out, res=other, workspace=dc2.workspace())
        U.compare(w, dc2.host(dc2.out), dc2.host(other), ref)
