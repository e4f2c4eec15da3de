"""GPU parity of BiasSoftmax (com.microsoft BiasSoftmax manifest): the HIP
path through the C ABI against the oracle's binary64 softmax of the binary32
sum data + bias, within the derived tolerance of gpu_util.SOFTMAX_TOL, for
every kernel family, skip (bias) form and the special values of the
definition."""
import numpy as np
import pytest

import transformer_residual_add_amd as T
from transformer_residual_add_amd import _lib as L
from transformer_residual_add_amd import workloads as W

import gpu_util as U

pytestmark = pytest.mark.gpu

MODES = ["exact", "outer", "inner"]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L.load()
    yield
    torch.cuda.synchronize()


def case(rows, hidden, dt, mode="exact", bias_rows=None, seed=1, data=W.normal(0, 2), bias=W.normal(0, 1)):
    if mode == "exact":
        bias_rows = None
    elif bias_rows is None:
        bias_rows = next(d for d in (4, 3, 2, 1) if rows % d == 0)
    return W.small_case(rows, hidden, dt, skip_rows=bias_rows, seed=seed, input_dist=data, skip_dist=bias,
                        op="bias_softmax", inner=mode == "inner")


def run_manual(w, x, b, variant=L.VARIANT_AUTO):
    """Run with hand-made data / bias arrays and compare with the oracle."""
    inputs = {"input": np.ascontiguousarray(x, dtype=w.np_dtype), "skip": np.ascontiguousarray(b, dtype=w.np_dtype),
              "gamma": None, "beta": None, "bias": None}
    return U.check_case(w, variant=variant, inputs=inputs)


# ------------------------------------------------------------ workloads --

@pytest.mark.parametrize("name", [n for n, w in W.EXTRA.items() if w.op == "bias_softmax"])
def test_softmax_workloads_all_rows(name):
    """Full size, automatic launch (the benchmark's), every row against the
    oracle; rows also sum to 1."""
    import torch

    w = W.EXTRA[name]
    code = L.F32 if w.dtype == "f32" else L.F16
    kernel = T.select_kernel(w.hidden, code, op=L.OP_BIAS_SOFTMAX, skip_mode=U.skip_mode(w), workspace=True)
    U.note(f"softmax workload {name}: rows={w.rows} block={w.hidden} {w.dtype} bias rows={w.skip_rows} {kernel}")
    # with a workspace, as the benchmark runs it (rows beyond the LDS split)
    dc, _ = U.check_case(w, workspace=True)
    s = dc.out.view(w.rows, w.hidden).double().sum(dim=1)
    assert torch.all((s - 1).abs() < (2e-3 if w.dtype == "f16" else 1e-5) * 8), "rows do not sum to 1"


# ------------------------------------------------------ shapes and forms --

HIDDEN = [1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 32, 63, 64, 77, 128, 197, 256, 512, 768, 1000, 1024, 1500, 2048, 4096,
          8192, 8196, 12288, 16384, 20000]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("mode", MODES)
def test_hidden_sizes(dt, hidden, mode):
    rows = 48 if hidden <= 4096 else 12
    w = case(rows, hidden, dt, mode, seed=hidden * 3 + MODES.index(mode))
    code = L.F32 if dt == "f32" else L.F16
    U.note(f"softmax {dt} H={hidden} {mode} kernel="
           f"{T.select_kernel(hidden, code, op=L.OP_BIAS_SOFTMAX, skip_mode=U.skip_mode(w))}")
    U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("variant", [L.VARIANT_GENERIC, L.VARIANT_ROWTILE, L.VARIANT_MULTIWAVE, L.VARIANT_LDSROW,
                                     L.VARIANT_ELEMENT, L.VARIANT_REGROW])
@pytest.mark.parametrize("hidden", [8, 64, 1024, 4096])
@pytest.mark.parametrize("mode", MODES)
def test_forced_variants(dt, variant, hidden, mode):
    w = case(40, hidden, dt, mode, bias_rows=8 if mode != "exact" else None, seed=hidden + variant)
    U.note(f"softmax variant {variant} {dt} H={hidden} {mode}")
    U.check_case(w, variant=variant)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("rows,bias_rows", [(96, 32), (96, 1), (96, 96), (1000, 8), (257, 257), (390, 13)])
@pytest.mark.parametrize("hidden", [4, 64, 768])
@pytest.mark.parametrize("mode", ["outer", "inner"])
def test_bias_reuse(dt, rows, bias_rows, hidden, mode):
    """Group sizes that do not split into whole row tiles, one bias row for
    all rows, one per row."""
    w = case(rows, hidden, dt, mode, bias_rows=bias_rows, seed=rows + bias_rows + hidden)
    U.note(f"softmax reuse {mode} {dt} rows={rows} bias rows={bias_rows} H={hidden}")
    U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("tiling", [(0, 1), (1, 0), (3, 1), (0, 2), (2, 2)], ids=lambda t: f"tpb{t[0]}_m{t[1]}")
@pytest.mark.parametrize("geom", [-1, 0, 12, 17, 18])
@pytest.mark.parametrize("mode", MODES)
def test_launch_configs(dt, tiling, geom, mode):
    w = case(203 if mode == "exact" else 210, 32 if dt == "f32" else 64, dt, mode, bias_rows=7,
             seed=geom + 100)
    if geom >= 0 and U.select(L.OP_BIAS_SOFTMAX, w.hidden, L.F32 if dt == "f32" else L.F16, U.skip_mode(w),
                              variant=L.VARIANT_GEOMETRY + geom) < 0:
        pytest.skip("geometry does not hold the row")
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=False)
    U.note(f"softmax config {dt} {mode} geometry={geom} tiling={tiling}")
    dc.run_config(geom, *tiling)
    U.compare(w, dc.host(dc.out), None, U.oracle_rows(w, inputs))


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("per", [0, 1, 3, 8])
@pytest.mark.parametrize("hidden", [64, 1024, 4096])
def test_bias_stationary_blocks(dt, per, hidden):
    """Cyclic bias rows kept stationary: each block keeps its tile of bias
    rows and walks `per` batches (0: the launcher's default), bias rows a
    whole number of tiles, a ragged last batch chunk (5 batches)."""
    w = case(5 * 64, hidden, dt, "outer", bias_rows=64, seed=hidden + per)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=False)
    U.note(f"softmax stationary {dt} H={hidden} per={per}")
    dc.run_config(-1, per, 2)
    U.compare(w, dc.host(dc.out), None, U.oracle_rows(w, inputs))


def test_large_cyclic_bias_automatic():
    """A per-head bias of 32 MiB (16384 rows of 1024 float16 keys) reused by 4
    batches: the automatic launch keeps it stationary; every row against the
    oracle."""
    w = case(4 * 16384, 1024, "f16", "outer", bias_rows=16384, seed=5)
    U.note("softmax large cyclic bias 65536 x 1024 f16, 16384 bias rows")
    dc, _ = U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_many_rows_packed(dt):
    """Many tiny rows (4- and 8-lane groups, many tiles per block)."""
    for hidden in (4, 8, 16, 32):
        w = case(100003 if hidden < 16 else 20011, hidden, dt, "exact", seed=hidden)
        U.note(f"softmax packed {dt} H={hidden} rows={w.rows}")
        U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_misaligned_pointers(dt):
    for hidden in (64, 1024, 77):
        w = case(20, hidden, dt, "outer", bias_rows=4, seed=hidden)
        U.note(f"softmax misaligned {dt} H={hidden}")
        U.check_case(w, offset_elems=1)


# --------------------------------------------- register-resident rows --

REGROW_HIDDEN = {"f32": [4100, 16384, 40960, 49152, 65536, 70000, 81920],
                 "f16": [8200, 40960, 65536, 100000, 128256, 131072, 140000, 151936, 163840]}


@pytest.mark.parametrize("dt,hidden", [(d, h) for d in ("f32", "f16") for h in REGROW_HIDDEN[d]])
@pytest.mark.parametrize("mode,bias_rows", [("exact", None), ("outer", 1), ("outer", 3), ("inner", 4), ("inner", 1)])
def test_regrow_long_rows(dt, hidden, mode, bias_rows):
    """Rows held in the registers of one 1024-lane block: partial last
    chunks per lane (ragged), the largest rows it holds, more rows than
    resident blocks (the persistent loop and its next-row loads), every bias
    form -- one bias row for all rows (parked in LDS) or several; the
    automatic choice beyond the LDS capacity."""
    rows = 300 if hidden <= 65536 else 264
    w = case(rows, hidden, dt, mode, bias_rows=bias_rows, seed=hidden + MODES.index(mode) + 7 * (bias_rows or 0))
    code = L.F32 if dt == "f32" else L.F16
    auto = T.select_kernel(hidden, code, op=L.OP_BIAS_SOFTMAX, skip_mode=U.skip_mode(w))
    # row tiles up to 2048 chunks, the LDS up to 40896 values, then registers
    assert (auto == f"softmax_regrow_{dt}") == (hidden > 40896), auto
    U.note(f"softmax regrow {dt} H={hidden} {mode} bias rows={bias_rows} rows={rows}")
    U.check_case(w, variant=L.VARIANT_REGROW)
    if hidden > 40896 and mode == "outer":
        U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_regrow_few_rows_and_in_place(dt):
    """Fewer rows than blocks; output over the data and over an exact bias."""
    hidden = 65536
    for rows, mode, bias_rows in ((1, "outer", 1), (3, "outer", 1), (1, "exact", None), (2, "exact", None),
                                  (5, "inner", 1)):
        w = case(rows, hidden, dt, mode, bias_rows=bias_rows, seed=rows)
        U.note(f"softmax regrow few rows {dt} rows={rows} {mode}")
        U.check_case(w, variant=L.VARIANT_REGROW)
    for over in ("data", "bias"):
        w = case(70, hidden, dt, "exact", seed=7)
        inputs = W.make_inputs(w)
        ref = U.oracle_rows(w, inputs)
        dc = U.DeviceCase(w, inputs, residual=False)
        U.note(f"softmax regrow in place over {over} {dt}")
        target = dc.x if over == "data" else dc.skip
        dc.run(L.VARIANT_REGROW, out=target)
        U.assert_out_close(dc.host(target), ref["y"], dt, tol=U.SOFTMAX_TOL)


# ------------------------------------------------------ special values --

SPECIAL_VARIANTS = [L.VARIANT_AUTO, L.VARIANT_GENERIC, L.VARIANT_MULTIWAVE, L.VARIANT_LDSROW, L.VARIANT_ELEMENT,
                    L.VARIANT_REGROW]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", [8, 64, 1024, 4096])
@pytest.mark.parametrize("variant", SPECIAL_VARIANTS)
def test_special_rows(dt, hidden, variant):
    """Row by row: a key-padding mask with -inf and with -10000; a row masked
    except one column; a row of -inf only (NaN); a NaN (NaN row); a +inf
    (NaN row); a masked suffix covering whole wavefronts; huge spread
    (underflowing terms); a large common offset; equal values."""
    code = L.F32 if dt == "f32" else L.F16
    if U.select(L.OP_BIAS_SOFTMAX, hidden, code, variant=variant) < 0:
        pytest.skip("family does not take this shape")
    rng = np.random.default_rng(hidden + variant)
    rows = 12
    x = rng.standard_normal((rows, hidden)) * 2
    b = np.zeros((rows, hidden))
    b[0, hidden // 3:] = -np.inf
    b[1, hidden // 2:] = -10000.0
    b[2, :] = -np.inf
    b[2, hidden - 1] = 0.0
    b[3, :] = -np.inf
    x[4, hidden // 2] = np.nan
    x[5, hidden - 1] = np.inf
    b[6, max(1, hidden // 8):] = -np.inf          # wavefronts 1.. of a multi-wave row fully masked
    x[7] = rng.standard_normal(hidden) * 40        # terms far below the maximum underflow
    x[8] = 1000.0 + rng.standard_normal(hidden) if dt == "f32" else 60000.0 + rng.standard_normal(hidden) * 8
    x[9] = 3.0
    b[10, 0] = -np.inf                             # only the first column masked
    x[11] = -1000.0 + rng.standard_normal(hidden)
    w = case(rows, hidden, dt, "exact", seed=0)
    U.note(f"softmax special {dt} H={hidden} variant={variant}")
    dc, ref = run_manual(w, x, b, variant)
    y = dc.host(dc.out)
    assert np.all(np.isnan(y[3])) and np.all(np.isnan(y[4])) and np.all(np.isnan(y[5]))
    assert np.all(y[0, hidden // 3:] == 0) and np.all(y[6, max(1, hidden // 8):] == 0)


def test_fully_masked_wavefronts_with_broadcast_mask():
    """Inner-broadcast key-padding mask whose kept prefix ends inside the
    first wavefront of a four-wavefront row: the other wavefronts see only
    -inf and must contribute zeros, not NaN."""
    hidden = 4096
    for dt in ("f32", "f16"):
        w = case(64, hidden, dt, "inner", bias_rows=4, seed=5)
        x = np.random.default_rng(3).standard_normal((64, hidden))
        b = np.zeros((4, hidden))
        for j, keep in enumerate((1, 100, 257, 4095)):
            b[j, keep:] = -np.inf
        for variant in (L.VARIANT_AUTO, L.VARIANT_MULTIWAVE, L.VARIANT_GENERIC, L.VARIANT_LDSROW, L.VARIANT_REGROW):
            U.note(f"softmax masked wavefronts {dt} variant={variant}")
            dc, _ = run_manual(w, x, b, variant)
            assert not np.isnan(dc.host(dc.out)).any()


# ------------------------------------------------------------ API paths --

def test_wrapper_shapes_and_axis():
    """bias_softmax on 4-D attention scores: key-padding mask (B,1,1,K) with
    inner reuse, per-head bias (1,H,Q,K) with outer reuse, axis -1 and 2,
    in place, and the empty cases of the contract."""
    import torch

    rng = np.random.default_rng(17)
    B, H, Q, K = 3, 4, 5, 24
    for dt, tdt in (("f32", torch.float32), ("f16", torch.float16)):
        npd = np.float32 if dt == "f32" else np.float16
        x = (rng.standard_normal((B, H, Q, K)) * 2).astype(npd)
        pad = np.zeros((B, 1, 1, K))
        pad[1, ..., 20:] = -np.inf
        pad[2, ..., 5:] = -10000.0
        pad = pad.astype(npd)
        pos = rng.standard_normal((1, H, Q, K)).astype(npd)
        xd = torch.from_numpy(x).cuda()
        for bias, inner in ((pad, True), (pos, False)):
            y = T.bias_softmax(xd, torch.from_numpy(bias).cuda(), inner, axis=-1)
            torch.cuda.synchronize()
            from oracle import oracle as O
            bias_rows = bias.reshape(-1, K)
            ref = O.bias_softmax(x.reshape(-1, K), bias_rows, inner)
            U.assert_out_close(y.cpu().numpy().reshape(-1, K), ref, dt, "wrapper", tol=U.SOFTMAX_TOL)
        # axis = 2: softmax over (Q, K) jointly, one bias row of Q*K per head
        hb = rng.standard_normal((H, Q, K)).astype(npd)
        y = T.bias_softmax(xd, torch.from_numpy(hb).cuda(), False, axis=2)
        torch.cuda.synchronize()
        ref = O.bias_softmax(x.reshape(-1, Q * K), hb.reshape(-1, Q * K), False)
        U.assert_out_close(y.cpu().numpy().reshape(-1, Q * K), ref, dt, "axis 2", tol=U.SOFTMAX_TOL)
        # in place over the data
        T.bias_softmax(xd, torch.from_numpy(pos).cuda(), False, axis=3, out=xd)
        torch.cuda.synchronize()
        ref = O.bias_softmax(x.reshape(-1, K), pos.reshape(-1, K), False)
        U.assert_out_close(xd.cpu().numpy().reshape(-1, K), ref, dt, "in place", tol=U.SOFTMAX_TOL)
    # empty data with empty bias: a no-op
    e = torch.empty((0, 4, 8), device="cuda")
    assert T.bias_softmax(e, torch.empty((0,), device="cuda"), True, axis=-1).shape == e.shape
    with pytest.raises(ValueError):
        T.bias_softmax(torch.zeros((4, 8), device="cuda"), torch.zeros((5,), device="cuda"), False, axis=1)
    with pytest.raises(T.SkiplnError) as err:   # 3 bias rows do not divide 4 rows
        T.bias_softmax(torch.zeros((4, 8), device="cuda"), torch.zeros((24,), device="cuda"), False, axis=1)
    assert err.value.status == L.ERR_SHAPE


def test_forced_variant_through_wrapper_matches_auto():
    import torch

    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((64, 1024)).astype(np.float32)).cuda()
    b = torch.from_numpy(rng.standard_normal((8, 1024)).astype(np.float32)).cuda()
    outs = [T.bias_softmax(x, b, True, axis=1, variant=v)
            for v in (L.VARIANT_AUTO, L.VARIANT_GENERIC, L.VARIANT_MULTIWAVE, L.VARIANT_LDSROW, L.VARIANT_REGROW)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.allclose(o, outs[0], rtol=4e-5, atol=1e-20)


def test_determinism_and_graph_replay():
    """Same bits on every launch, eager and replayed from a HIP graph."""
    import torch

    w = W.EXTRA["softmax_relpos_64x12x128x128_f32"].with_(shape=(4 * 12 * 128, 128))
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=False)
    dc.run()
    first = dc.out.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dc.run(stream=s.cuda_stream)
        dc.run(stream=s.cuda_stream)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dc.run(stream=s.cuda_stream)
    for _ in range(3):
        dc.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc.out.view(torch.int32), first.view(torch.int32))
    U.compare(w, dc.host(dc.out), None, U.oracle_rows(w, inputs))
