"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Normalized output within (1e-5 + 1e-5|y|) for float32 and
(2e-3 + 2e-3|y|) for float16 of the oracle's binary64 value; the residual
(input_skip_bias_sum) bit for bit."""
import numpy as np
import pytest

import transformer_residual_add_amd as T
from transformer_residual_add_amd import _lib as L
from transformer_residual_add_amd import workloads as W

import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L.load()  # raises if libskipln.so cannot be loaded: no silent fallback
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------ workloads --

@pytest.mark.parametrize("name", W.ORDER[:3])
def test_workload_all_rows(name):
    w = W.WORKLOADS[name]
    U.note(f"workload {name}: rows={w.rows} H={w.hidden} {w.dtype}")
    U.check_case(w)


ORACLE_BLOCK = 4096  # rows per oracle call in the full-size comparison


# The two largest configurations, the benchmark's full-size root-mean-square
# and BiasAdd workloads, and 2 GiB layer norms that take the single-tile form.
FULL_SIZE = list(W.ORDER[3:]) + ["rms_rows65536_h8192_f16", "biasadd_64x512x4096_f16", "rows65536_h4096_f16",
                                   "rows131072_h2048_f16", "rows16384_h16384_f16", "rows16384_h12288_f32",
                                   "rows16384_h14336_f32"]


@pytest.mark.parametrize("name", FULL_SIZE)
def test_workload_full_size_every_row(name):
    """Full-size run in the benchmark's launch configuration, every row
    compared with the oracle: the normalized output within tolerance, the
    residual (when emitted) and BiasAdd's output bit for bit.  The oracle runs
    in blocks of rows on the host's cores while the device result is copied
    back block by block."""
    import torch

    w = W.get(name)
    U.note(f"workload {name}: generating rows={w.rows} H={w.hidden} {w.dtype}")
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=w.residual)
    mode = L.SKIP_BROADCAST if w.broadcast else L.SKIP_EXACT
    kernel = T.select_kernel(w.hidden, L.F32 if w.dtype == "f32" else L.F16, skip_mode=mode, op=U.OPS[w.op],
                             rows=w.rows)
    U.note(f"workload {name}: launching {kernel}")
    dc.run()
    torch.cuda.synchronize()
    U.note(f"workload {name}: comparing all {w.rows} rows with the oracle")
    out = dc.out.view(w.rows, w.hidden)
    res = dc.res.view(w.rows, w.hidden) if dc.res is not None else None
    threads = W.default_threads()
    for r0 in range(0, w.rows, ORACLE_BLOCK):
        r1 = min(w.rows, r0 + ORACLE_BLOCK)
        part = dict(inputs)
        part["input"] = inputs["input"][r0:r1]
        if not w.broadcast:
            part["skip"] = inputs["skip"][r0:r1]
        ref = U.oracle_rows(w, part, row_offset=r0, threads=threads)
        if w.op == "bias_add":
            U.assert_bits_equal(out[r0:r1].cpu().numpy(), ref["y"], f"bias_add out rows {r0}:{r1}")
        else:
            U.assert_out_close(out[r0:r1].cpu().numpy(), ref["y"], w.dtype, f"out rows {r0}:{r1}")
        if res is not None:
            U.assert_bits_equal(res[r0:r1].cpu().numpy(), ref["residual"], f"residual rows {r0}:{r1}")


STORE_THROUGH_BYTES = 512 << 20  # launches writing this much store with the system-scope policy


@pytest.mark.parametrize("dt,hidden,residual,op", [("f16", 1000, True, "layer_norm"), ("f32", 999, True, "layer_norm"),
                                                    ("f16", 1024, False, "simplified"),
                                                    ("f32", 1000, False, "bias_add")],
                         ids=["elem_f16_ln", "elem_f32_ln", "chunk_f16_rms", "elem_f32_biasadd"])
@pytest.mark.parametrize("side", ["below", "above"])
def test_store_policies_at_the_threshold(dt, hidden, residual, op, side):
    """Launches just below and just above the output size where the row
    tiles switch to system-scope stores, for chunk and element-wise tiles:
    sampled row blocks against the oracle, every row of the last block."""
    import torch

    itemsize = 4 if dt == "f32" else 2
    per_row = hidden * itemsize * (2 if residual else 1)
    rows = STORE_THROUGH_BYTES // per_row + (1 if side == "above" else -1)
    assert (rows * per_row >= STORE_THROUGH_BYTES) == (side == "above")
    w = W.small_case(rows, hidden, dt, beta=op != "bias_add", bias=True, residual=residual, eps=1e-5,
                     seed=hidden + rows % 97, op=op)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=w.residual)
    code = L.F32 if dt == "f32" else L.F16
    U.note(f"store policy {side}: {op} {dt} rows={rows} H={hidden} "
           f"{T.select_kernel(hidden, code, op=U.OPS[op])}")
    dc.run()
    torch.cuda.synchronize()
    out = dc.out.view(w.rows, w.hidden)
    res = dc.res.view(w.rows, w.hidden) if dc.res is not None else None
    n_blocks = -(-w.rows // W.BLOCK_ROWS)
    for b in sorted({0, n_blocks // 3, n_blocks - 1}):
        r0, r1 = b * W.BLOCK_ROWS, min(w.rows, (b + 1) * W.BLOCK_ROWS)
        part = {k: (None if v is None else v[r0:r1] if k in ("input", "skip") else v) for k, v in inputs.items()}
        ref = U.oracle_rows(w, part, row_offset=r0)
        U.compare(w, out[r0:r1].cpu().numpy(), None if res is None else res[r0:r1].cpu().numpy(), ref)


# ------------------------------------------------------ flags and shapes --

FLAG_SETS = [(bool(m & 1), bool(m & 2), bool(m & 4), bool(m & 8)) for m in range(16)]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", [64, 768, 1000, 4096])
@pytest.mark.parametrize("flags", FLAG_SETS, ids=lambda f: "b%d_bi%d_r%d_bc%d" % tuple(map(int, f)))
def test_flag_matrix(dt, hidden, flags):
    beta, bias, residual, bcast = flags
    w = W.small_case(48, hidden, dt, skip_rows=8 if bcast else None, beta=beta, bias=bias, residual=residual,
                     eps=1e-5 if dt == "f16" else 1e-12, seed=hidden + 17 * sum(1 << i for i, f in enumerate(flags) if f))
    U.note(f"flags {dt} H={hidden} beta={beta} bias={bias} residual={residual} bcast={bcast}")
    U.check_case(w)


HIDDEN = [1, 2, 3, 4, 7, 8, 12, 16, 63, 64, 65, 96, 127, 128, 255, 256, 768, 1000, 1024, 1536, 2048, 2049, 3072,
          4096, 6144, 8192, 12288, 16384, 20000]


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", HIDDEN)
def test_hidden_sizes(dt, hidden):
    w = W.small_case(37, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=hidden)
    U.note(f"hidden {dt} H={hidden} kernel={T.select_kernel(hidden, L.F32 if dt == 'f32' else L.F16)}")
    U.check_case(w)


ROWTILE_GEOMETRIES = range(L.load_tune().skipln_tune_rowtile_geometries())
ELEMENT_GEOMETRIES = range(L.load_tune().skipln_tune_element_geometries())


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("geom", ROWTILE_GEOMETRIES)
@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_add", "bias_softmax"])
def test_every_geometry(dt, geom, ragged, op):
    """Each row-tile geometry, for each operation, at its full capacity and
    one chunk short of it, with a ragged last tile of rows."""
    op_code = U.OPS[op]
    v = 4 if dt == "f32" else 8
    code = L.F32 if dt == "f32" else L.F16
    # capacity in chunks: the largest hidden size the geometry accepts
    cap = 0
    for hv in range(1, 4097):
        if U.select(L.OP_LAYER_NORM, hv * v, code, variant=L.VARIANT_GEOMETRY + geom) < 0:
            break
        cap = hv
    hidden = (cap - 1 if ragged and cap > 1 else cap) * v
    name = L.kernel_name(U.select(op_code, hidden, code, variant=L.VARIANT_GEOMETRY + geom))
    g = int(name.split("_g")[1].split("_")[0])
    block = int(name.split("_b")[1]) if "_b" in name else max(256, g)
    rpb = block // g
    rows = 3 * rpb + 1
    w = W.small_case(rows, hidden, dt, beta=True, bias=ragged, residual=True, eps=1e-5, seed=geom * 7 + ragged,
                     op=op)
    U.note(f"geometry {geom} ({name}) H={hidden} rows={rows}")
    U.check_case(w, variant=L.VARIANT_GEOMETRY + geom)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("geom", ROWTILE_GEOMETRIES)
@pytest.mark.parametrize("form_cap", [(1, 0), (1, 3), (0, -1)], ids=lambda f: f"form{f[0]}_cap{f[1]}")
@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_add", "bias_softmax"])
def test_kernel_forms(dt, geom, form_cap, op):
    """Both kernel forms of one-tile-per-block launches at every geometry
    (the single-tile form with and without a blocks-per-CU limit), one chunk
    short of capacity, a ragged last tile of rows, a broadcast skip on the
    normalizations."""
    form, cap = form_cap
    v = 4 if dt == "f32" else 8
    code = L.F32 if dt == "f32" else L.F16
    chunks = 0
    for hv in range(1, 4097):
        if U.select(L.OP_LAYER_NORM, hv * v, code, variant=L.VARIANT_GEOMETRY + geom) < 0:
            break
        chunks = hv
    hidden = max(1, chunks - 1) * v
    name = L.kernel_name(U.select(U.OPS[op], hidden, code, variant=L.VARIANT_GEOMETRY + geom))
    g = int(name.split("_g")[1].split("_")[0])
    block = int(name.split("_b")[1]) if "_b" in name else max(256, g)
    rows = 3 * (block // g) + 1
    bcast = op in ("layer_norm", "simplified")
    w = W.small_case(rows, hidden, dt, skip_rows=1 if bcast else None, beta=True, bias=True, residual=True,
                     eps=1e-5, seed=geom * 11 + form * 3 + cap + 1, op=op)
    inputs = W.make_inputs(w)
    U.note(f"form {form} cap {cap} geometry {geom} ({name}) {op} H={hidden} rows={rows}")
    dc = U.DeviceCase(w, inputs, residual=w.residual)
    dc.run_form(geom, form, cap)
    U.compare(w, dc.host(dc.out), dc.host(dc.res) if w.residual else None, U.oracle_rows(w, inputs))


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("geom", ROWTILE_GEOMETRIES)
@pytest.mark.parametrize("op", ["layer_norm", "bias_softmax"])
def test_single_tile_blocks_per_cu(dt, geom, op):
    """The single-tile form's blocks-per-CU limit (set through the launch's
    LDS) holds a compute unit to exactly min(limit, what its registers allow)
    for every limit from 1 to 8; the table's limit never exceeds the
    registers' count."""
    tune = L.load_tune()
    code = L.F32 if dt == "f32" else L.F16
    bpc = lambda form, cap: tune.skipln_tune_blocks_per_cu(U.OPS[op], code, geom, form, cap)
    free = bpc(1, 0)
    assert free >= 1 and bpc(0, -1) >= 1
    for cap in range(1, 9):
        assert bpc(1, cap) == min(cap, free), (cap, free)
    assert 1 <= bpc(1, -1) <= free


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("geom", ELEMENT_GEOMETRIES)
@pytest.mark.parametrize("shape", ["full", "odd", "short"])
@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_add", "bias_softmax"])
def test_every_element_geometry(dt, geom, shape, op):
    """Each element-wise row-tile geometry, for each operation: at its full
    capacity, at an odd length just below, and at a quarter (idle lanes),
    with a ragged last tile of rows and a broadcast skip."""
    code = L.F32 if dt == "f32" else L.F16
    cap = 0
    for h in (16384, 8192, 4096, 2048, 1024, 512, 256, 128, 64, 32, 16, 8, 4, 2, 1):
        if U.select(L.OP_LAYER_NORM, h, code, variant=L.VARIANT_ELEMENT_GEOMETRY + geom) >= 0:
            cap = h
            break
    hidden = {"full": cap, "odd": max(1, cap - 1), "short": max(1, cap // 4 + 1)}[shape]
    variant = L.VARIANT_ELEMENT_GEOMETRY + geom
    name = L.kernel_name(U.select(U.OPS[op], hidden, code, variant=variant))
    g = int(name.split("_g")[1].split("_")[0])
    block = int(name.split("_b")[1]) if "_b" in name else max(256, g)
    rows = 3 * (block // g) + 1 if hidden <= 4096 else 9
    bcast = op != "bias_add" and rows % 3 == 0
    w = W.small_case(rows, hidden, dt, skip_rows=3 if bcast else None, beta=True, bias=shape != "full",
                     residual=True, eps=1e-5, seed=geom * 5 + len(shape), op=op)
    U.note(f"element geometry {geom} ({name}) {op} H={hidden} rows={rows}")
    U.check_case(w, variant=variant)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("tiling", [(0, 1), (1, 0), (3, 1), (0, 2), (2, 2)], ids=lambda t: f"tpb{t[0]}_m{t[1]}")
@pytest.mark.parametrize("geom_hidden", [(0, 3), (5, 77), (8, 1000), (4, 63)], ids=lambda g: f"e{g[0]}_h{g[1]}")
def test_element_launch_configs(dt, tiling, geom_hidden):
    geom, hidden = geom_hidden
    w = W.small_case(203, hidden, dt, skip_rows=7, beta=True, bias=True, residual=True, eps=1e-5, seed=31)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=True)
    U.note(f"element config {dt} geometry={geom} H={hidden} tiling={tiling}")
    dc.run_config(L.VARIANT_ELEMENT_GEOMETRY + geom, *tiling)
    ref = U.oracle_rows(w, inputs)
    U.assert_out_close(dc.host(dc.out), ref["y"], dt)
    U.assert_bits_equal(dc.host(dc.res), ref["residual"])


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("variant", [L.VARIANT_GENERIC, L.VARIANT_MULTIWAVE, L.VARIANT_ROWTILE, L.VARIANT_ELEMENT])
@pytest.mark.parametrize("hidden", [64, 1024, 4096])
def test_forced_variants(dt, variant, hidden):
    w = W.small_case(40, hidden, dt, skip_rows=8, beta=True, bias=True, residual=True, eps=1e-5, seed=3)
    U.note(f"variant {variant} {dt} H={hidden}")
    U.check_case(w, variant=variant)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", [64, 1024, 999])
def test_misaligned_pointers_use_generic(dt, hidden):
    w = W.small_case(20, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=11)
    U.note(f"misaligned {dt} H={hidden}")
    U.check_case(w, offset_elems=1)


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_many_rows_small_hidden(dt):
    """Many row tiles per persistent block."""
    w = W.small_case(100003, 64, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=5)
    U.note(f"many rows {dt}")
    U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("tiling", [(0, 1), (1, 0), (1, 1), (3, 0), (3, 1), (7, 0), (1000, 1), (0, 0), (0, 2),
                                    (1, 2), (2, 2), (5, 2), (1000, 2)],
                         ids=lambda t: f"tpb{t[0]}_m{t[1]}")
@pytest.mark.parametrize("geom_hidden", [(-1, 1024), (0, 48), (7, 4000), (13, 768)],
                         ids=lambda g: f"g{g[0]}_h{g[1]}")
def test_launch_configs(dt, tiling, geom_hidden):
    """Every tiling (persistent, contiguous, strided, more tiles per block
    than exist) gives the same, correct result."""
    geom, hidden = geom_hidden
    if dt == "f16" and hidden % 8:
        hidden += 8 - hidden % 8
    w = W.small_case(203, hidden, dt, skip_rows=7, beta=True, bias=True, residual=True, eps=1e-5, seed=13)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=True)
    U.note(f"config {dt} geometry={geom} H={hidden} tiling={tiling}")
    dc.run_config(geom, *tiling)
    ref = U.oracle_rows(w, inputs)
    U.assert_out_close(dc.host(dc.out), ref["y"], dt)
    U.assert_bits_equal(dc.host(dc.res), ref["residual"])


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("geom,hidden,S,batches", [(7, 4096, 8, 13), (12, 512, 6, 5), (0, 64, 32, 5), (0, 64, 24, 3),
                                                    (7, 2048, 1, 9), (15, 768, 5, 4)])
@pytest.mark.parametrize("tpb", [0, 1, 3])
def test_skip_stationary_tiles(dt, geom, hidden, S, batches, tpb):
    """Broadcast skip with blocks that keep their skip rows across batches,
    including multi-row tiles and a skip row count that does not split into
    whole tiles (falls back to strided)."""
    w = W.small_case(S * batches, hidden, dt, skip_rows=S if S * batches != S else None, beta=True, bias=True,
                     residual=True, eps=1e-5, seed=S + batches)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=True)
    U.note(f"stationary {dt} geometry={geom} H={hidden} S={S} N={batches} tpb={tpb}")
    dc.run_config(geom, tpb, L.TILE_SKIP_STATIONARY)
    ref = U.oracle_rows(w, inputs)
    U.assert_out_close(dc.host(dc.out), ref["y"], dt)
    U.assert_bits_equal(dc.host(dc.res), ref["residual"])


def test_launch_config_errors():
    w = W.small_case(8, 64, "f32", residual=True)
    dc = U.DeviceCase(w, W.make_inputs(w), residual=True)
    with pytest.raises(T.SkiplnError) as e:
        dc.run_config(0, -1, 0)
    assert e.value.status == L.ERR_SHAPE
    with pytest.raises(T.SkiplnError) as e:
        dc.run_config(L.load_tune().skipln_tune_rowtile_geometries(), 1, 0)
    assert e.value.status == L.ERR_VARIANT
    with pytest.raises(T.SkiplnError) as e:
        dc.run_config(-2, 1, 0)
    assert e.value.status == L.ERR_VARIANT
    with pytest.raises(T.SkiplnError) as e:
        dc.run_config(0, 1, 3)
    assert e.value.status == L.ERR_VARIANT


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (64 << 20) + 48])
def test_streaming_copy(nbytes):
    import torch

    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    L.check(L.load_tune().skipln_tune_copy(dst.data_ptr(), src.data_ptr(), nbytes, None), "skipln_tune_copy")
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert L.load_tune().skipln_tune_copy(dst.data_ptr() + 8, src.data_ptr(), 16, None) == L.ERR_SHAPE
    assert L.load_tune().skipln_tune_copy(dst.data_ptr(), src.data_ptr(), 24, None) == L.ERR_SHAPE


def test_stream_probe_outputs():
    """The streaming probe's outputs: a copy, the XOR of two inputs, the copy
    plus one, and the chunk index when nothing is read -- in address order and
    with tiles dealt to the XCDs in granules (a permutation of the tiles, with
    a ragged last tile and a partial last round), with either store policy."""
    import torch

    lib = L.load_tune()
    n = (1 << 20) + 48
    a = torch.randint(0, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    b = torch.randint(0, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    c, d = torch.zeros_like(a), torch.zeros_like(a)
    for blk, u, g, t in ((64, 1, 1, 0), (256, 4, 1, 1), (1024, 1, 1, 0), (1024, 4, 1, 1), (64, 1, 2, 0), (64, 1, 3, 1),
                         (64, 4, 16, 0), (256, 1, 5, 1)):
        c.zero_(), d.zero_()
        L.check(lib.skipln_tune_stream(a.data_ptr(), None, c.data_ptr(), d.data_ptr(), n, blk, u, g, t, None),
                "skipln_tune_stream")
        torch.cuda.synchronize()
        assert torch.equal(c, a) and torch.equal(d, a + 1), (blk, u, g, t)
    for g, t in ((1, 0), (4, 1)):
        c.zero_()
        L.check(lib.skipln_tune_stream(a.data_ptr(), b.data_ptr(), c.data_ptr(), None, n, 256, 1, g, t, None),
                "skipln_tune_stream")
        torch.cuda.synchronize()
        assert torch.equal(c, a ^ b)
    idx = torch.arange(n // 16, dtype=torch.int32, device="cuda")
    for g, t in ((1, 1), (7, 0)):
        c.fill_(-1)
        L.check(lib.skipln_tune_stream(None, None, c.data_ptr(), None, n, 64, 4, g, t, None), "skipln_tune_stream")
        torch.cuda.synchronize()
        assert torch.equal(c.view(-1, 4)[:, 0], idx) and not c.view(-1, 4)[:, 1:].any()
    before = c.clone()
    L.check(lib.skipln_tune_stream(a.data_ptr(), b.data_ptr(), None, None, n, 1024, 4, 2, 0, None), "skipln_tune_stream")
    torch.cuda.synchronize()
    assert torch.equal(c, before)


# ------------------------------------------------- simplified and BiasAdd --

@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", [1, 7, 64, 768, 1000, 1024, 4096, 8192, 20000])
@pytest.mark.parametrize("flags", [(True, True, True, False), (False, False, False, False),
                                   (True, False, True, True), (False, True, False, True)],
                         ids=lambda f: "b%d_bi%d_r%d_bc%d" % tuple(map(int, f)))
def test_simplified(dt, hidden, flags):
    beta, bias, residual, bcast = flags
    w = W.small_case(24, hidden, dt, skip_rows=4 if bcast else None, beta=beta, bias=bias, residual=residual,
                     eps=1e-6, seed=hidden + 5, op="simplified")
    U.note(f"simplified {dt} H={hidden} flags={flags}")
    U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("hidden", [1, 3, 8, 64, 768, 1000, 1024, 4096, 8192, 20000])
@pytest.mark.parametrize("rows", [1, 37, 1000])
def test_bias_add(dt, hidden, rows):
    w = W.small_case(rows, hidden, dt, seed=hidden + rows, op="bias_add")
    U.note(f"bias_add {dt} H={hidden} rows={rows}")
    U.check_case(w)


@pytest.mark.parametrize("op", ["simplified", "bias_add"])
@pytest.mark.parametrize("variant", [L.VARIANT_GENERIC, L.VARIANT_MULTIWAVE, L.VARIANT_ROWTILE])
@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_new_ops_forced_variants(op, variant, dt):
    w = W.small_case(40, 1024, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=8, op=op)
    U.check_case(w, variant=variant)


@pytest.mark.parametrize("misalign", [0, 1], ids=["aligned", "misaligned"])
@pytest.mark.parametrize("rows_hidden", [(600, 64), (40, 8200), (12, 40000), (6, 65536), (6, 65537)],
                         ids=lambda t: f"{t[0]}x{t[1]}")
@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_add", "bias_softmax"])
def test_generic_both_forms(op, dt, rows_hidden, misalign):
    """The generic kernel in its 16-byte-chunk form (aligned rows of whole
    chunks) and its element form (misaligned tensors, or a row that ends
    inside a chunk), forced, for every operation: more rows than resident
    blocks (a block's reduction slots reused), rows with fewer chunks than
    lanes, ragged batches of chunks, long rows far from zero mean."""
    rows, hidden = rows_hidden
    kw = dict(input_dist=W.normal(100.0, 1)) if op in ("layer_norm", "simplified") else {}
    if op == "bias_softmax":
        w = W.small_case(rows, hidden, dt, skip_rows=2, op=op, seed=rows + hidden + misalign)
    else:
        w = W.small_case(rows, hidden, dt, skip_rows=None if op == "bias_add" else 2, beta=True, bias=True,
                         residual=True, eps=1e-5, seed=rows + hidden + misalign, op=op, **kw)
    U.note(f"generic {op} {dt} {rows}x{hidden} misalign={misalign}")
    U.check_case(w, variant=L.VARIANT_GENERIC, offset_elems=misalign)


@pytest.mark.parametrize("op", ["simplified", "bias_add"])
def test_new_ops_misaligned(op):
    w = W.small_case(20, 1024, "f16", beta=True, bias=True, residual=True, eps=1e-5, seed=9, op=op)
    U.check_case(w, offset_elems=1)


@pytest.mark.parametrize("name", [n for n, w in W.EXTRA.items() if w.op != "bias_softmax"])
def test_extra_workloads(name):
    w = W.EXTRA[name]
    U.note(f"workload {name}")
    if w.rows * w.hidden > 50_000_000:
        rows = min(2048, 50_000_000 // w.hidden)
        w = w.with_(shape=(rows, w.hidden) if len(w.shape) == 2 else (4,) + w.shape[1:],
                    skip_shape=(rows, w.hidden) if len(w.shape) == 2 else (4,) + w.shape[1:])
    U.check_case(w)


def test_bias_add_in_place_and_wrapper():
    import torch

    w = W.small_case(64, 768, "f32", seed=3, op="bias_add")
    inputs = W.make_inputs(w)
    ref = U.oracle_rows(w, inputs)
    x = torch.from_numpy(inputs["input"]).cuda().view(4, 16, 768)
    sk = torch.from_numpy(inputs["skip"]).cuda().view(4, 16, 768)
    b = torch.from_numpy(inputs["bias"]).cuda()
    y = T.bias_add(x, b, sk)
    torch.cuda.synchronize()
    U.assert_bits_equal(y.cpu().numpy().reshape(64, 768), ref["y"])
    T.bias_add(x, b, sk, out=x)  # in place over X
    torch.cuda.synchronize()
    U.assert_bits_equal(x.cpu().numpy().reshape(64, 768), ref["y"])
    with pytest.raises(ValueError):
        T.bias_add(x, b, sk[:2])
    with pytest.raises(ValueError):
        T.bias_add(x, b[:5], sk)


def test_simplified_wrapper():
    import torch

    w = W.small_case(32, 1024, "f16", beta=False, bias=True, residual=True, eps=1e-6, seed=4, op="simplified")
    inputs = W.make_inputs(w)
    ref = U.oracle_rows(w, inputs)
    d = {k: (None if v is None else torch.from_numpy(v).cuda()) for k, v in inputs.items()}
    out, res = T.skip_layer_norm(d["input"], d["skip"], d["gamma"], None, d["bias"], epsilon=w.eps,
                                 return_residual=True, simplified=True)
    torch.cuda.synchronize()
    U.assert_out_close(out.cpu().numpy(), ref["y"], "f16")
    U.assert_bits_equal(res.cpu().numpy(), ref["residual"])


# ------------------------------------------------------------- long rows --

LDS_F32 = [4, 64, 1000, 4096, 8196, 12288, 16384, 20000, 32768, 40896]
LDS_F16 = [8, 64, 1000, 8192, 16392, 24576, 32768, 40896]


@pytest.mark.parametrize("op", ["layer_norm", "simplified"])
@pytest.mark.parametrize("dt_hidden", [("f32", h) for h in LDS_F32] + [("f16", h) for h in LDS_F16],
                         ids=lambda t: f"{t[0]}_h{t[1]}")
@pytest.mark.parametrize("flags", [(True, True, True, False), (False, False, False, True)],
                         ids=lambda f: "b%d_bi%d_r%d_bc%d" % tuple(map(int, f)))
def test_long_rows_lds_staged(op, dt_hidden, flags):
    """The LDS-staged kernel, forced, from a few chunks (ragged lanes) up to
    the 160 KiB row limit."""
    dt, hidden = dt_hidden
    beta, bias, residual, bcast = flags
    rows = 6 if hidden > 16384 else 21
    w = W.small_case(rows, hidden, dt, skip_rows=3 if bcast else None, beta=beta, bias=bias, residual=residual,
                     eps=1e-5, seed=hidden + 1, op=op)
    U.note(f"ldsrow {op} {dt} H={hidden} flags={flags}")
    U.check_case(w, variant=L.VARIANT_LDSROW)


REGNORM_HIDDEN = {"f32": [36868, 40960, 41000, 45056, 50000, 57344, 61444, 65536],
                  "f16": [32776, 40960, 41000, 45056, 50000, 57344, 61448, 65536]}


@pytest.mark.parametrize("op", ["layer_norm", "simplified"])
@pytest.mark.parametrize("dt_hidden", [(d, h) for d in ("f32", "f16") for h in REGNORM_HIDDEN[d]],
                         ids=lambda t: f"{t[0]}_h{t[1]}")
@pytest.mark.parametrize("flags", ["all", "bare", "bcast"])
def test_register_resident_normalizations(op, dt_hidden, flags):
    """Rows held in the registers of one 1024-lane block, forced: every
    compiled slab count, rows ending inside a slab, with and without beta,
    bias and residual, exact and broadcast skip."""
    dt, hidden = dt_hidden
    rows = 6 if flags == "bcast" else 7
    w = W.small_case(rows, hidden, dt, skip_rows=3 if flags == "bcast" else None, beta=flags != "bare",
                     bias=flags != "bare", residual=flags != "bare", eps=1e-5, seed=hidden % 97, op=op)
    U.note(f"regnorm {op} {dt} H={hidden} {flags}")
    U.check_case(w, variant=L.VARIANT_REGROW)


@pytest.mark.parametrize("dt,hidden,mu", [("f32", 65536, 1000.0), ("f16", 61448, 100.0), ("f32", 45056, 100.0)])
def test_register_resident_normalizations_many_rows_far_from_zero(dt, hidden, mu):
    """More rows than resident blocks (the persistent loop and its next-row
    loads) with a mean far from zero (the statistics' shift), forced."""
    w = W.small_case(600, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=3,
                     input_dist=W.normal(mu, 1))
    U.note(f"regnorm many rows {dt} H={hidden} mu={mu}")
    U.check_case(w, variant=L.VARIANT_REGROW)


def test_register_resident_normalizations_special_values():
    """A NaN stays in its row; a constant row with eps = 0 is NaN (0/0)."""
    w = W.small_case(5, 45056, "f32", beta=True, bias=True, residual=True, eps=0.0, seed=4)
    inputs = W.make_inputs(w)
    inputs["input"][1, 7] = np.nan
    inputs["input"][2, :] = 3.0
    inputs["skip"][2, :] = 0.0
    inputs["bias"][:] = 0.0
    U.note("regnorm special values")
    U.check_case(w, variant=L.VARIANT_REGROW, inputs=inputs)


@pytest.mark.parametrize("dt,hidden,rows", [("f16", 65536, 300), ("f32", 49152, 64)])
def test_register_resident_normalizations_auto(dt, hidden, rows):
    """The automatic choice takes the register-resident rows where they win."""
    code = L.F32 if dt == "f32" else L.F16
    assert T.select_kernel(hidden, code, rows=rows).startswith("regrow_")
    w = W.small_case(rows, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=hidden + rows)
    U.note(f"regnorm auto {dt} H={hidden} rows={rows}")
    U.check_case(w)


@pytest.mark.parametrize("dt,hidden", [("f32", 12288), ("f32", 40896), ("f16", 32768)])
def test_long_rows_auto(dt, hidden):
    w = W.small_case(300 if hidden < 20000 else 64, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5,
                     seed=hidden, input_dist=W.normal(100, 1))
    code = L.F32 if dt == "f32" else L.F16
    assert T.select_kernel(hidden, code).startswith("ldsrow_")
    U.note(f"ldsrow auto {dt} H={hidden}")
    U.check_case(w)


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("mu", [100.0, 1000.0])
@pytest.mark.parametrize("hidden", [64, 768, 4096, 12288])
@pytest.mark.parametrize("variant", [L.VARIANT_AUTO, L.VARIANT_MULTIWAVE, L.VARIANT_GENERIC, L.VARIANT_LDSROW,
                                     L.VARIANT_ELEMENT, L.VARIANT_SPAN])
def test_large_offset_rows(dt, mu, hidden, variant):
    """Rows whose mean is far from zero (variance cancellation) in every
    kernel family, within the binary32 tolerance."""
    code = L.F32 if dt == "f32" else L.F16
    if U.select(L.OP_LAYER_NORM, hidden, code, variant=variant) < 0:
        pytest.skip("family does not take this shape")
    w = W.small_case(40, hidden, dt, skip_rows=8, beta=True, bias=True, residual=True, eps=1e-5, seed=int(mu) + hidden,
                     input_dist=W.normal(mu, 1))
    U.note(f"offset {mu} {dt} H={hidden} variant={variant}")
    U.check_case(w, variant=variant)


def test_long_rows_reject_tiling():
    w = W.small_case(4, 20000, "f32", residual=True)
    dc = U.DeviceCase(w, W.make_inputs(w), residual=True)
    assert U.select(L.OP_LAYER_NORM, 20000, L.F32, variant=L.VARIANT_LDSROW) >= 0
    with pytest.raises(T.SkiplnError) as e:
        dc.run_config(-1, 1, 1)  # no row-tile geometry holds 5000 chunks
    assert e.value.status == L.ERR_UNSUPPORTED


# ------------------------------------------------------------ edge cases --

def test_rows_zero_is_noop():
    import torch

    w = W.small_case(0, 64, "f32", residual=True)
    dc = U.DeviceCase(w, W.make_inputs(w), residual=True)
    dc.run()
    torch.cuda.synchronize()


@pytest.mark.parametrize("variant_hidden", [(L.VARIANT_AUTO, 1024), (L.VARIANT_GENERIC, 1024),
                                            (L.VARIANT_MULTIWAVE, 1024), (L.VARIANT_LDSROW, 12288),
                                            (L.VARIANT_ELEMENT, 1000), (L.VARIANT_AUTO, 1000),
                                            (L.VARIANT_REGROW, 65536), (L.VARIANT_AUTO, 49152)],
                         ids=lambda t: f"v{t[0]}_h{t[1]}")
@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("op", ["layer_norm", "simplified"])
def test_in_place(variant_hidden, dt, op):
    """out over input and residual over the (exact) skip, in every family:
    no lane may read a value another lane has already overwritten."""
    variant, hidden = variant_hidden
    w = W.small_case(33, hidden, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=21,
                     input_dist=W.normal(50, 1), op=op)
    inputs = W.make_inputs(w)
    ref = U.oracle_rows(w, inputs)
    dc = U.DeviceCase(w, inputs, residual=True)
    U.note(f"in place {op} {dt} variant {variant} H={hidden}")
    dc.run(variant, out=dc.x, res=dc.skip)
    U.assert_out_close(dc.host(dc.x), ref["y"], dt)
    U.assert_bits_equal(dc.host(dc.skip), ref["residual"])


@pytest.mark.parametrize("variant", [L.VARIANT_AUTO, L.VARIANT_GENERIC])
def test_nan_stays_in_its_row(variant):
    w = W.small_case(16, 768, "f32", beta=True, bias=True, residual=True, eps=1e-5, seed=4)
    inputs = W.make_inputs(w)
    inputs["input"][5, 17] = np.nan
    inputs["input"][9, 0] = np.inf
    dc, ref = U.check_case(w, variant=variant, inputs=inputs)
    out = dc.host(dc.out)
    assert np.isnan(out[5]).all() and np.isnan(out[9]).all()
    assert np.isfinite(np.delete(out, [5, 9], axis=0)).all()


@pytest.mark.parametrize("variant", [L.VARIANT_AUTO, L.VARIANT_GENERIC, L.VARIANT_MULTIWAVE])
def test_constant_row_with_zero_eps(variant):
    w = W.small_case(8, 128, "f32", beta=True, residual=True, eps=0.0, seed=9)
    inputs = W.make_inputs(w)
    inputs["input"][2] = 3.0
    inputs["skip"][2] = 0.5
    dc, ref = U.check_case(w, variant=variant, inputs=inputs)
    assert np.isnan(dc.host(dc.out)[2]).all()


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_single_column(dt):
    w = W.small_case(9, 1, dt, beta=True, bias=True, residual=True, eps=1e-5, seed=2)
    dc, ref = U.check_case(w)
    assert np.array_equal(dc.host(dc.out).astype(np.float64)[:, 0],
                          np.repeat(W.make_inputs(w)["beta"].astype(np.float64), 9))


def test_deterministic_reruns():
    w = W.WORKLOADS["rows16384_h1024_f16"].with_(shape=(4096, 1024), skip_shape=(4096, 1024))
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=True)
    dc.run()
    a = dc.host(dc.out).copy()
    ra = dc.host(dc.res).copy()
    dc.run()
    assert np.array_equal(a.view(np.uint16), dc.host(dc.out).view(np.uint16))
    assert np.array_equal(ra.view(np.uint16), dc.host(dc.res).view(np.uint16))


def test_non_default_stream():
    import torch

    w = W.small_case(64, 2048, "f32", beta=True, bias=True, residual=True, eps=1e-5, seed=6)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dc.run(stream=s.cuda_stream)
    s.synchronize()
    ref = U.oracle_rows(w, inputs)
    U.assert_out_close(dc.host(dc.out), ref["y"], "f32")
    U.assert_bits_equal(dc.host(dc.res), ref["residual"])


def test_more_than_2_to_the_32_rows():
    """Row indices past 32 bits (2^32 + 8 rows of one value, float16): the
    64-bit row and broadcast-skip paths.  With H = 1 the output is beta
    exactly; the residual must equal x + skip[r mod 4] bit for bit."""
    import torch

    rows, S = (1 << 32) + 8, 4
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(rows, 1, device="cuda", dtype=torch.float16, generator=g)
    skip = torch.randn(S, 1, device="cuda", dtype=torch.float16, generator=g)
    gamma = torch.full((1,), 1.5, device="cuda", dtype=torch.float16)
    beta = torch.full((1,), 0.25, device="cuda", dtype=torch.float16)
    out = torch.empty_like(x)
    res = torch.empty_like(x)
    torch.cuda.synchronize()
    U.note(f"rows={rows} H=1 f16 inputs ready; launching {T.select_kernel(1, L.F16, skip_mode=L.SKIP_BROADCAST)}")
    T.forward_raw(x.data_ptr(), skip.data_ptr(), L.SKIP_BROADCAST, S, gamma.data_ptr(), beta.data_ptr(), None,
                  out.data_ptr(), res.data_ptr(), rows, 1, 1e-5, L.F16)
    torch.cuda.synchronize()
    U.note("kernel done; checking")
    assert bool((out == 0.25).all()), "H = 1 must give beta"
    step = 1 << 28
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        want = (x[r0:r1].float() + skip.repeat((r1 - r0) // S, 1).float()).half()
        assert torch.equal(res[r0:r1].view(torch.int16), want.view(torch.int16)), f"residual rows {r0}:{r1}"
    # the last rows, past 2^32, by hand
    for r in (rows - 1, rows - 5, (1 << 32) + 1):
        assert res[r].item() == (x[r].float() + skip[r % S].float()).half().item()


def test_concurrent_host_threads_and_streams():
    """Eight host threads, each with its own stream and problem (every
    operation and kernel family), launching at once: each result equals the
    oracle (the library keeps no mutable state besides an attribute cache)."""
    import threading

    import torch

    cases = [W.small_case(64, 1024, "f16", beta=True, bias=True, residual=True, eps=1e-5, seed=61),
             W.small_case(40, 768, "f32", skip_rows=8, residual=True, eps=1e-5, seed=62),
             W.small_case(33, 1000, "f32", bias=True, residual=True, eps=1e-5, seed=63, op="simplified"),
             W.small_case(48, 12288, "f32", beta=True, residual=True, eps=1e-5, seed=64),
             W.small_case(64, 4096, "f16", seed=65, op="bias_add"),
             W.small_case(96, 77, "f16", skip_rows=3, seed=66, op="bias_softmax", inner=True),
             W.small_case(256, 512, "f32", skip_rows=4, seed=67, op="bias_softmax"),
             W.small_case(8, 65536, "f32", beta=True, residual=True, eps=1e-5, seed=68)]
    devs = []
    for w in cases:
        inputs = W.make_inputs(w)
        devs.append((w, inputs, U.DeviceCase(w, inputs, residual=w.residual)))
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(len(devs))

    def work(dc):
        try:
            s = torch.cuda.Stream()
            start.wait()
            for _ in range(5):
                dc.run(stream=s.cuda_stream, workspace=True)
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(dc,)) for _, _, dc in devs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for w, inputs, dc in devs:
        U.note(f"concurrent {w.name}")
        U.compare(w, dc.host(dc.out), dc.host(dc.res) if w.residual else None, U.oracle_rows(w, inputs))


@pytest.mark.parametrize("name", ["bert_base_8x128x768_f32", "bcast_64x512x4096_f32"])
def test_graph_replay_matches_eager(name):
    """Captured into a HIP graph, every replay (with eager work and
    synchronizations in between) equals the eager launch on the same input."""
    import torch

    w = W.WORKLOADS[name]
    if w.rows > 4096:
        w = w.with_(shape=(8,) + w.shape[1:])
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=True)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        dc.run(stream=torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        dc.x.mul_(0.5).add_(float(rep))  # eager work between replays: new input
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_out, got_res = dc.out.clone(), dc.res.clone()
        dc.out.fill_(float("nan"))
        dc.res.fill_(float("nan"))
        dc.run()
        torch.cuda.synchronize()
        assert torch.equal(got_out, dc.out) and torch.equal(got_res, dc.res), f"replay {rep} differs"


def test_error_enqueues_nothing():
    import torch

    w = W.small_case(4, 64, "f32", residual=True)
    dc = U.DeviceCase(w, W.make_inputs(w), residual=True)
    with pytest.raises(T.SkiplnError) as e:
        T.forward_raw(dc.x.data_ptr(), dc.skip.data_ptr(), L.SKIP_EXACT, 0, dc.gamma.data_ptr(), None, None,
                      dc.out.data_ptr(), dc.res.data_ptr(), w.rows, w.hidden, -1.0, L.F32)
    assert e.value.status == L.ERR_EPS
    torch.cuda.synchronize()
    assert torch.isnan(dc.out).all() and torch.isnan(dc.res).all()


# ------------------------------------------------------- Python wrapper --

@pytest.mark.parametrize("skip_form", ["exact", "1SH", "SH"])
def test_python_wrapper_rank3(skip_form):
    import torch

    N, S, H = 4, 16, 768
    w = W.Workload(name="wrapper", shape=(N, S, H), dtype="f32",
                   skip_shape=(N, S, H) if skip_form == "exact" else (S, H), input_dist=W.normal(0, 1),
                   skip_dist=W.normal(0, 1), bias_dist=W.normal(0, 0.1), residual=True, eps=1e-12, seed=44)
    inputs = W.make_inputs(w)
    x = torch.from_numpy(inputs["input"]).cuda().view(N, S, H)
    sk = torch.from_numpy(inputs["skip"]).cuda()
    sk = sk.view(N, S, H) if skip_form == "exact" else (sk.view(1, S, H) if skip_form == "1SH" else sk.view(S, H))
    g, b, bi = (torch.from_numpy(inputs[k]).cuda() for k in ("gamma", "beta", "bias"))
    out, res = T.skip_layer_norm(x, sk, g, b, bi, epsilon=w.eps, return_residual=True)
    torch.cuda.synchronize()
    ref = U.oracle_rows(w, inputs)
    U.assert_out_close(out.cpu().numpy().reshape(-1, H), ref["y"], "f32")
    U.assert_bits_equal(res.cpu().numpy().reshape(-1, H), ref["residual"])
    assert out.shape == x.shape and res.shape == x.shape


def test_python_wrapper_rejects_bad_inputs():
    import torch

    x = torch.zeros(2, 8, 64, device="cuda")
    g = torch.ones(64, device="cuda")
    with pytest.raises(TypeError):
        T.skip_layer_norm(x, x.half(), g)
    with pytest.raises(ValueError):
        T.skip_layer_norm(x, torch.zeros(3, 64, device="cuda"), g)
    with pytest.raises(ValueError):
        T.skip_layer_norm(x, x, torch.ones(63, device="cuda"))
    with pytest.raises(T.SkiplnError):
        T.skip_layer_norm(x, x, g, epsilon=-1.0)
    with pytest.raises(TypeError):
        T.skip_layer_norm(x.double(), x.double(), g.double())


def _subnormal_rows(w, seed):
    """float16 inputs whose rows 0..5 hold subnormal values (multiples of
    2^-24 below 2^-14, exact in binary16): rows 0-1 all of x, skip and bias
    subnormal; rows 2-3 subnormal x with normal skip; rows 4-5 subnormal x
    and bias with a zero skip."""
    rng = np.random.default_rng(seed)
    inputs = W.make_inputs(w)
    h = w.hidden

    def sub(n):
        m = rng.integers(-1023, 1024, size=n)
        m[m == 0] = 1
        return (m.astype(np.float64) * 2.0 ** -24).astype(np.float16)

    x, s = inputs["input"], inputs["skip"]
    for r in range(6):
        x[r] = sub(h)
    s[0], s[1] = sub(h), sub(h)
    s[4] = 0
    s[5] = 0
    if inputs.get("bias") is not None:
        inputs["bias"][:] = sub(h)
    assert np.all(np.abs(x[:6].astype(np.float64)) < 2.0 ** -14)
    return inputs


@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_add"])
@pytest.mark.parametrize("variant_hidden", [(L.VARIANT_AUTO, 1000), (L.VARIANT_GENERIC, 1000),
                                            (L.VARIANT_MULTIWAVE, 1000), (L.VARIANT_ROWTILE, 1000),
                                            (L.VARIANT_ELEMENT, 1000), (L.VARIANT_ROWTILE, 8192),
                                            (L.VARIANT_LDSROW, 20000), (L.VARIANT_SPLITROW, 20000)],
                         ids=lambda t: f"v{t[0]}_h{t[1]}")
def test_float16_subnormals(op, variant_hidden):
    """binary16 subnormal data, skip and bias are widened exactly: the
    residual (and BiasAdd's output) is bit-exact, and with eps = 0 rows made
    only of subnormals normalize to O(1) values (a kernel that flushed them
    would see a zero row, zero variance and NaN)."""
    variant, hidden = variant_hidden
    if op == "bias_add" and variant in (L.VARIANT_LDSROW, L.VARIANT_SPLITROW):
        pytest.skip("BiasAdd has no row statistics, so no LDS-staged or split-row kernel")
    w = W.small_case(24, hidden, "f16", beta=True, bias=True, residual=op != "bias_add", eps=0.0,
                     seed=hidden + 3, op=op)
    inputs = _subnormal_rows(w, seed=hidden)
    U.note(f"float16 subnormals {op} variant {variant} H={hidden}")
    dc, ref = U.check_case(w, variant=variant, inputs=inputs, workspace=variant == L.VARIANT_SPLITROW or None)
    out = dc.host(dc.out).astype(np.float64)
    assert np.isfinite(out).all()
    if op != "bias_add":
        assert np.abs(out[:6]).max() > 0.5


@pytest.mark.parametrize("op", ["layer_norm", "simplified", "bias_add"])
@pytest.mark.parametrize("dt,rows,hidden", [("f32", 1024, 768), ("f16", 1024, 768), ("f16", 5, 1024),
                                            ("f32", 37, 4096), ("f16", 300, 8192)],
                         ids=lambda v: str(v))
def test_streamed_first_tile_matches_cached(op, dt, rows, hidden):
    """A launch of one wave of resident blocks with one tile each reads an
    exact skip with non-temporal loads (a kernel instantiation of its own);
    launches whose blocks walk two tiles read it through the caches.  The
    arithmetic is the same, so the outputs agree bit for bit, and with the
    oracle."""
    w = W.small_case(rows, hidden, dt, beta=True, bias=True, residual=op != "bias_add", eps=1e-5,
                     seed=rows + hidden, op=op)
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=w.residual)
    U.note(f"streamed first tile {op} {dt} {rows}x{hidden}")
    dc.run()
    out_auto = dc.host(dc.out).copy()
    res_auto = dc.host(dc.res).copy() if w.residual else None
    ref = U.oracle_rows(w, inputs)
    U.compare(w, out_auto, res_auto, ref)
    for tpb, strided in [(2, 1), (2, 0)]:
        dc.out.fill_(float("nan"))
        if w.residual:
            dc.res.fill_(float("nan"))
        dc.run_config(-1, tpb, strided)
        U.assert_bits_equal(dc.host(dc.out), out_auto, f"out, {tpb} tiles per block")
        if w.residual:
            U.assert_bits_equal(dc.host(dc.res), res_auto, f"residual, {tpb} tiles per block")


@pytest.mark.parametrize("hidden", [131072, 128256], ids=["whole_slabs", "ragged_last_slab"])
def test_register_resident_store_policies(hidden):
    """The register-resident softmax above the store threshold, one bias row:
    system-scope stores for rows of whole 16 KiB slabs (131072 float16
    values), non-temporal ones for rows with a ragged last slab; sampled row
    blocks against the oracle."""
    import torch

    rows = STORE_THROUGH_BYTES // (hidden * 2) + 1
    w = W.small_case(rows, hidden, "f16", skip_rows=1, seed=hidden % 1000, input_dist=W.normal(0, 2),
                     skip_dist=W.normal(0, 1), op="bias_softmax")
    inputs = W.make_inputs(w)
    dc = U.DeviceCase(w, inputs, residual=False)
    name = T.select_kernel(hidden, L.F16, op=U.OPS["bias_softmax"], skip_mode=L.SKIP_BROADCAST)
    assert name.startswith("softmax_regrow_"), name
    U.note(f"register-resident store policy: rows={rows} H={hidden} {name}")
    dc.run()
    torch.cuda.synchronize()
    out = dc.out.view(w.rows, w.hidden)
    n_blocks = -(-w.rows // W.BLOCK_ROWS)
    for b in sorted({0, n_blocks // 2, n_blocks - 1}):
        r0, r1 = b * W.BLOCK_ROWS, min(w.rows, (b + 1) * W.BLOCK_ROWS)
        part = dict(inputs)
        part["input"] = inputs["input"][r0:r1]
        ref = U.oracle_rows(w, part, row_offset=r0)
        U.compare(w, out[r0:r1].cpu().numpy(), None, ref)


def _random_case(rng):
    """One random workload: operation, type, rows, hidden size (ragged,
    chunk-multiple, power of two, long), optional tensors, skip form."""
    op = str(rng.choice(["layer_norm", "simplified", "bias_add", "bias_softmax"], p=[0.4, 0.2, 0.2, 0.2]))
    dt = str(rng.choice(["f32", "f16"]))
    kind = int(rng.integers(0, 4))
    if kind == 0:
        hidden = int(rng.integers(1, 300))
    elif kind == 1:
        hidden = int(rng.integers(1, 600)) * (4 if dt == "f32" else 8)
    elif kind == 2:
        hidden = 1 << int(rng.integers(4, 14))
    else:
        hidden = int(rng.integers(8000, 40000))
    rows = int(rng.integers(1, 200 if hidden < 8000 else 40))
    skip_rows = None
    if rng.random() < 0.3 and op != "bias_add":  # BiasAdd's skip has X's shape
        divisors = [d for d in range(1, rows + 1) if rows % d == 0 and d < rows]
        if divisors:
            skip_rows = int(rng.choice(divisors))
    inner = op == "bias_softmax" and skip_rows is not None and bool(rng.random() < 0.5)
    w = W.small_case(rows, hidden, dt, skip_rows=skip_rows, beta=bool(rng.random() < 0.7),
                     bias=bool(rng.random() < 0.6), residual=bool(rng.random() < 0.6) and op != "bias_add",
                     eps=float(rng.choice([1e-5, 1e-12, 1e-3])), seed=int(rng.integers(1, 1 << 30)), op=op,
                     inner=inner)
    offset = int(rng.choice([0, 0, 0, 1, 3]))
    return w, offset


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes(seed):
    """Twenty-five random workloads per seed (operation, type, rows, hidden size,
    optional tensors, skip form, misaligned pointers), each through the
    automatic kernel choice and compared with the oracle row by row."""
    rng = np.random.default_rng(20_000 + seed)
    for i in range(25):
        w, offset = _random_case(rng)
        U.note(f"random seed={seed} case={i}: {w.op} {w.dtype} shape={w.shape} skip={w.skip_shape} "
               f"residual={w.residual} offset={offset}")
        inputs = W.make_inputs(w)
        dc = U.DeviceCase(w, inputs, residual=w.residual, offset_elems=offset)
        dc.run()
        ref = U.oracle_rows(w, inputs)
        U.compare(w, dc.host(dc.out), dc.host(dc.res) if w.residual else None, ref)


@pytest.mark.parametrize("op", ["layer_norm", "simplified"])
def test_large_broadcast_skip_automatic(op):
    """A 16 MiB skip (2048 rows of 4096 float16 values) broadcast over 5
    batches: the automatic launch keeps the skip rows stationary and walks up
    to 8 batches per block (here all 5); every row against the oracle."""
    w = W.small_case(5 * 2048, 4096, "f16", skip_rows=2048, beta=True, bias=True, residual=True, eps=1e-5,
                     seed=77, op=op)
    U.note(f"large broadcast skip {op} (5, 2048, 4096) f16")
    U.check_case(w)
