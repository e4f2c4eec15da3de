"""GPU parity of the span row tiles: rows that are not whole 16-byte chunks,
with every tensor 16-byte aligned, read as the aligned chunks their bytes
touch.  Each geometry and operation against the oracle (normalized outputs
and softmax within the float tolerances of gpu_util, residual and BiasAdd
bit for bit), at the geometry's longest row, a middle and a tiny one, with
ragged tiles of rows, exact and broadcast skips, in place, special values,
and the automatic choice over odd row lengths."""
import numpy as np
import pytest

import transformer_residual_add_amd as T
from transformer_residual_add_amd import _lib as L
from transformer_residual_add_amd import workloads as W

import gpu_util as U

pytestmark = pytest.mark.gpu

SPAN_GEOMETRIES = range(L.load_tune().skipln_tune_span_geometries())


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L.load()
    yield
    torch.cuda.synchronize()


def _shape_of(op: str, code: int, geom: int):
    """(lanes per row, chunks per lane, block) of span geometry `geom`."""
    name = L.kernel_name(U.select(U.OPS[op], 1, code, variant=L.VARIANT_SPAN_GEOMETRY + geom))
    g = int(name.split("_g")[1].split("_")[0])
    ch = int(name.split("_c")[1].split("_")[0])
    block = int(name.split("_b")[1]) if "_b" in name else max(256, g)
    return g, ch, block


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("geom", SPAN_GEOMETRIES)
@pytest.mark.parametrize("shape", ["full", "mid", "tiny"])
@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_add", "bias_softmax"])
def test_every_span_geometry(dt, geom, shape, op):
    """The longest row the geometry holds (not a whole number of chunks),
    about half of it, and three values; three and a bit tiles of rows; a
    broadcast skip (cyclic for the normalizations and the 'tiny' softmax,
    grouped for the 'mid' softmax); mean 50 on the longest normalization
    rows."""
    code = L.F32 if dt == "f32" else L.F16
    sz = 4 if dt == "f32" else 2
    v = 16 // sz
    g, ch, block = _shape_of(op, code, geom)
    hmax = (g * ch - 1) * 16 // sz
    assert (hmax * sz + 15) // 16 + 1 <= g * ch
    full = hmax if hmax % v else hmax - 1
    hidden = {"full": full, "mid": max(1, full // 2) | 1, "tiny": 3}[shape]
    rows = 3 * (block // g) + 3
    seed = geom * 13 + len(shape) + hidden
    if op == "bias_softmax":
        w = W.small_case(rows, hidden, dt, skip_rows=None if shape == "full" else 3, op=op, inner=shape == "mid",
                         seed=seed)
    elif op == "bias_add":
        w = W.small_case(rows, hidden, dt, bias=True, op=op, seed=seed)
    else:
        kw = dict(input_dist=W.normal(50, 1)) if shape == "full" else {}
        w = W.small_case(rows, hidden, dt, skip_rows=3 if shape == "mid" else None, beta=shape != "tiny",
                         bias=shape != "tiny", residual=True, eps=1e-5, seed=seed, op=op, **kw)
    U.note(f"span geometry {geom} (g{g} c{ch}) {op} {dt} {shape} H={hidden} rows={rows}")
    U.check_case(w, variant=L.VARIANT_SPAN_GEOMETRY + geom)


AUTO_LENGTHS = [1, 2, 3, 5, 7, 9, 13, 31, 33, 63, 77, 127, 197, 255, 257, 511, 769, 1001, 1500, 2047, 3001, 4095,
                8191, 12289]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", AUTO_LENGTHS)
@pytest.mark.parametrize("op", ["layer_norm", "bias_add", "bias_softmax"])
def test_span_automatic_choice(dt, hidden, op):
    """Rows that are not whole chunks take the span tiles automatically where
    they measured faster (element-wise tiles elsewhere) and match the
    oracle."""
    code = L.F32 if dt == "f32" else L.F16
    sz = 4 if dt == "f32" else 2
    if hidden * sz % 16 == 0:
        pytest.skip("whole chunks: the chunk row tiles")
    name = T.select_kernel(hidden, code, op=U.OPS[op])
    touched = (hidden * sz + 15) // 16 + 1
    # exact skip or bias: BiasSoftmax rows touching 8 to 2048 chunks, BiasAdd
    # rows touching 64 to 2048; never the normalizations
    lo = {"bias_softmax": 8, "bias_add": 64}.get(op)
    span = lo is not None and lo <= touched <= 2048
    assert ("span_" in name) == span, name
    if op != "bias_add":
        bname = T.select_kernel(hidden, code, op=U.OPS[op], skip_mode=L.SKIP_BROADCAST)
        assert "span_" not in bname, bname
    rows = 40 if hidden < 4096 else 8
    if op == "bias_softmax":
        w = W.small_case(rows, hidden, dt, op=op, seed=hidden)
    elif op == "bias_add":
        w = W.small_case(rows, hidden, dt, bias=True, op=op, seed=hidden)
    else:
        w = W.small_case(rows, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=hidden)
    U.note(f"span auto {op} {dt} H={hidden} -> {name}")
    U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", [3, 77, 1001])
def test_span_in_place(dt, hidden):
    """out over input and residual over the exact skip: a row's end chunks are
    shared with its neighbours, whose lanes may already have written their
    own elements of them."""
    w = W.small_case(37, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=hidden + 1,
                     input_dist=W.normal(20, 1))
    inputs = W.make_inputs(w)
    ref = U.oracle_rows(w, inputs)
    dc = U.DeviceCase(w, inputs, residual=True)
    U.note(f"span in place {dt} H={hidden}")
    dc.run(L.VARIANT_SPAN, out=dc.x, res=dc.skip)
    U.assert_out_close(dc.host(dc.x), ref["y"], dt)
    U.assert_bits_equal(dc.host(dc.skip), ref["residual"])


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", [77, 121, 197])
def test_span_softmax_in_place(dt, hidden):
    """Softmax written over its data: on rows of 8 and 16 lanes the chunk two
    rows share is spliced from both rows' results and stored whole by the
    later row, after both rows have read it."""
    w = W.small_case(8 * 64 + 5, hidden, dt, op="bias_softmax", seed=hidden + 2)
    inputs = W.make_inputs(w)
    ref = U.oracle_rows(w, inputs)
    dc = U.DeviceCase(w, inputs, residual=False)
    U.note(f"span softmax in place {dt} H={hidden}")
    dc.run(L.VARIANT_SPAN, out=dc.x)
    U.assert_out_close(dc.host(dc.x), ref["y"], dt)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_span_softmax_special_values(dt):
    """-inf keys (a padding mask), a row of -inf only (NaN), a NaN and a +inf
    (their rows NaN), and every other row finite, in rows of 197 keys."""
    w = W.small_case(12, 197, dt, skip_rows=3, op="bias_softmax", inner=False, seed=11)
    inputs = W.make_inputs(w)
    inputs["input"][1, 150:] = -np.inf
    inputs["input"][4, :] = -np.inf
    inputs["skip"][1, :] = 0  # row 4 reads bias row 1: all -inf stays all -inf
    inputs["input"][7, 5] = np.nan
    inputs["input"][10, 196] = np.inf
    U.note(f"span softmax special values {dt}")
    dc, ref = U.check_case(w, variant=L.VARIANT_SPAN, inputs=inputs)
    out = dc.host(dc.out)
    assert np.isnan(out[4]).all() and np.isnan(out[7]).all() and np.isnan(out[10]).all()
    assert (out[1, 150:] == 0).all()
    assert np.isfinite(np.delete(out, [4, 7, 10], axis=0)).all()


def test_span_rows_of_one_value():
    """Rows of one float16 value (eight rows per chunk, each written by its own
    lane), a broadcast skip of four rows: H = 1 gives beta, the residual is
    x + skip bit for bit.  (Launches past 2^32 work-items, whose blocks walk
    several tiles, are test_parity_gpu's test_more_than_2_to_the_32_rows.)"""
    w = W.small_case(4096 + 4, 1, "f16", skip_rows=4, beta=True, bias=False, residual=True, eps=1e-5, seed=3)
    U.note("span H=1 rows=4100")
    dc, ref = U.check_case(w, variant=L.VARIANT_SPAN)
    assert np.array_equal(dc.host(dc.out).astype(np.float64)[:, 0],
                          np.repeat(W.make_inputs(w)["beta"].astype(np.float64), w.rows))
