"""The C ABIs on the CPU: libskipln.so and libskipln_tune.so load, export
exactly the functions their headers declare (include/skipln.h,
include/skipln_tune.h), their enums match the Python binding, and every
argument check is reachable from the host (the validate, select and
workspace-size entry points make no HIP call)."""
import math
import os
import re
import subprocess

import pytest

from transformer_residual_add_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skipln.h")
TUNE_HEADER = os.path.join(ROOT, "include", "skipln_tune.h")


def _read(path):
    with open(path) as fh:
        return fh.read()


def _declared(text):
    return set(re.findall(r"^SKIPLN_API\s+(?:int|int64_t|const char\*)\s+(skipln_\w+)\s*\(", text, re.M))


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


@pytest.mark.parametrize("header,signatures,loader,path", [
    (HEADER, L.SIGNATURES, L.load, L.LIB_PATH),
    (TUNE_HEADER, L.TUNE_SIGNATURES, L.load_tune, L.TUNE_LIB_PATH),
], ids=["operator", "tune"])
def test_header_functions_are_the_only_exports(header, signatures, loader, path):
    declared = _declared(_read(header))
    assert declared, "no declarations found"
    assert declared == set(signatures), f"binding and header differ: {declared ^ set(signatures)}"
    lib = loader()
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    assert _exported(path) == declared, f"exports differ from the header: {_exported(path) ^ declared}"


def test_operator_surface():
    """The operator library's surface: the operator, its argument checks,
    the three operations beside it, the workspace form, status strings."""
    assert set(L.SIGNATURES) == {
        "skipln_forward", "skipln_validate", "skipln_status_string", "skipln_version",
        "skipln_forward_simplified", "skipln_bias_add", "skipln_bias_softmax",
        "skipln_forward_ws", "skipln_workspace_bytes", "skipln_forward_ws_static"}
    assert L.load().skipln_version() == 2


def test_validate_takes_the_forward_arguments():
    """skipln_validate takes skipln_forward's arguments, the stream aside."""
    text = _read(HEADER)

    def params(name):
        m = re.search(r"SKIPLN_API int " + name + r"\((.*?)\);", text, re.S)
        return [p.strip() for p in " ".join(m.group(1).split()).split(",")]

    fwd, val = params("skipln_forward"), params("skipln_validate")
    assert fwd[-1] == "skipln_stream_t stream"
    norm = lambda ps: [p.replace("const ", "") for p in ps]
    assert norm(val) == norm(fwd[:-1])


def test_header_enums_match_binding():
    vals = {k: int(v) for k, v in re.findall(r"(SKIPLN_\w+)\s*=\s*(-?\d+)", _read(HEADER) + _read(TUNE_HEADER))}
    expect = {
        "SKIPLN_F32": L.F32, "SKIPLN_F16": L.F16,
        "SKIPLN_SKIP_EXACT": L.SKIP_EXACT, "SKIPLN_SKIP_BROADCAST": L.SKIP_BROADCAST,
        "SKIPLN_SKIP_BROADCAST_INNER": L.SKIP_BROADCAST_INNER,
        "SKIPLN_OK": L.OK, "SKIPLN_ERR_NULL": L.ERR_NULL, "SKIPLN_ERR_SHAPE": L.ERR_SHAPE,
        "SKIPLN_ERR_DTYPE": L.ERR_DTYPE, "SKIPLN_ERR_MODE": L.ERR_MODE, "SKIPLN_ERR_EPS": L.ERR_EPS,
        "SKIPLN_ERR_ALIAS": L.ERR_ALIAS, "SKIPLN_ERR_UNSUPPORTED": L.ERR_UNSUPPORTED,
        "SKIPLN_ERR_LAUNCH": L.ERR_LAUNCH, "SKIPLN_ERR_DEVICE": L.ERR_DEVICE,
        "SKIPLN_ERR_VARIANT": L.ERR_VARIANT, "SKIPLN_ERR_OP": L.ERR_OP, "SKIPLN_ERR_WORKSPACE": L.ERR_WORKSPACE,
        "SKIPLN_OP_LAYER_NORM": L.OP_LAYER_NORM, "SKIPLN_OP_SIMPLIFIED": L.OP_SIMPLIFIED,
        "SKIPLN_OP_BIAS_ADD": L.OP_BIAS_ADD, "SKIPLN_OP_BIAS_SOFTMAX": L.OP_BIAS_SOFTMAX,
        "SKIPLN_VARIANT_AUTO": L.VARIANT_AUTO, "SKIPLN_VARIANT_GENERIC": L.VARIANT_GENERIC,
        "SKIPLN_VARIANT_ROWTILE": L.VARIANT_ROWTILE, "SKIPLN_VARIANT_MULTIWAVE": L.VARIANT_MULTIWAVE,
        "SKIPLN_VARIANT_LDSROW": L.VARIANT_LDSROW, "SKIPLN_VARIANT_SPLITROW": L.VARIANT_SPLITROW,
        "SKIPLN_VARIANT_ELEMENT": L.VARIANT_ELEMENT,
        "SKIPLN_VARIANT_REGROW": L.VARIANT_REGROW, "SKIPLN_VARIANT_ELEMENT_GEOMETRY": L.VARIANT_ELEMENT_GEOMETRY,
        "SKIPLN_VARIANT_GEOMETRY": L.VARIANT_GEOMETRY, "SKIPLN_VARIANT_SPAN": L.VARIANT_SPAN,
        "SKIPLN_VARIANT_SPAN_GEOMETRY": L.VARIANT_SPAN_GEOMETRY,
        "SKIPLN_TILE_CONTIGUOUS": L.TILE_CONTIGUOUS, "SKIPLN_TILE_STRIDED": L.TILE_STRIDED,
        "SKIPLN_TILE_SKIP_STATIONARY": L.TILE_SKIP_STATIONARY,
        "SKIPLN_STORE_AUTO": L.STORE_AUTO, "SKIPLN_STORE_STREAM": L.STORE_STREAM,
        "SKIPLN_STORE_THROUGH": L.STORE_THROUGH,
    }
    assert vals == expect


def test_status_strings():
    for st in range(0, 13):
        assert L.status_string(st) not in ("", "unknown status")
    assert L.status_string(99) == "unknown status"


# Disjoint fake device addresses: validate never dereferences them.
IN, SK, GA, BE, BI, OUT, RES = (0x100000 * k for k in range(1, 8))


def V(input=IN, skip=SK, mode=0, skip_rows=0, gamma=GA, beta=BE, bias=BI, out=OUT, res=RES, rows=4, hidden=8,
      eps=1e-5, dtype=0, op=L.OP_LAYER_NORM):
    """The layer norm's checks through the operator library's skipln_validate;
    the other operations' through the tuning library's op-aware validate
    (the two must agree on the layer norm)."""
    args = (input, skip, mode, skip_rows, gamma, beta, bias, out, res, rows, hidden, eps, dtype)
    tuned = L.load_tune().skipln_tune_validate(op, *args)
    if op == L.OP_LAYER_NORM:
        st = L.load().skipln_validate(*args)
        assert st == tuned
        return st
    return tuned


def test_validate_accepts_good_arguments():
    assert V() == L.OK
    assert V(beta=None, bias=None, res=None) == L.OK
    assert V(mode=1, skip_rows=2) == L.OK
    assert V(dtype=1) == L.OK
    assert V(eps=0.0) == L.OK and V(eps=math.inf) == L.OK


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), L.ERR_DTYPE),
    (dict(dtype=-1), L.ERR_DTYPE),
    (dict(mode=2), L.ERR_MODE),
    (dict(eps=-1e-7), L.ERR_EPS),
    (dict(eps=math.nan), L.ERR_EPS),
    (dict(hidden=0), L.ERR_SHAPE),
    (dict(hidden=-3), L.ERR_SHAPE),
    (dict(hidden=2 ** 31), L.ERR_SHAPE),
    (dict(rows=-1), L.ERR_SHAPE),
    (dict(rows=2 ** 62, hidden=8), L.ERR_SHAPE),
    (dict(mode=1, skip_rows=0), L.ERR_SHAPE),
    (dict(mode=1, skip_rows=3), L.ERR_SHAPE),   # 4 rows not a multiple of 3
    (dict(mode=1, skip_rows=-2), L.ERR_SHAPE),
    (dict(input=None), L.ERR_NULL),
    (dict(skip=None), L.ERR_NULL),
    (dict(gamma=None), L.ERR_NULL),
    (dict(out=None), L.ERR_NULL),
    (dict(out=IN + 4), L.ERR_ALIAS),            # partial overlap with input
    (dict(out=SK, mode=1, skip_rows=2), L.ERR_ALIAS),  # broadcast skip is read by many rows
    (dict(out=SK + 32), L.ERR_ALIAS),
    (dict(out=GA), L.ERR_ALIAS),
    (dict(out=BE), L.ERR_ALIAS),
    (dict(res=BI), L.ERR_ALIAS),
    (dict(res=OUT), L.ERR_ALIAS),
    (dict(res=OUT + 64), L.ERR_ALIAS),
])
def test_validate_rejects(kw, status):
    assert V(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(op=4), L.ERR_OP),
    (dict(op=-1), L.ERR_OP),
    (dict(op=L.OP_SIMPLIFIED, gamma=None), L.ERR_NULL),
    (dict(op=L.OP_SIMPLIFIED), L.OK),
    (dict(op=L.OP_BIAS_ADD), L.OK),
    (dict(op=L.OP_BIAS_ADD, gamma=None, beta=None, res=None, eps=-1.0), L.OK),  # ignored by BiasAdd
    (dict(op=L.OP_BIAS_ADD, bias=None), L.ERR_NULL),
    (dict(op=L.OP_BIAS_ADD, mode=1, skip_rows=2), L.ERR_MODE),
    (dict(op=L.OP_BIAS_ADD, out=BI), L.ERR_ALIAS),
    (dict(op=L.OP_BIAS_ADD, out=IN), L.OK),
    (dict(op=L.OP_BIAS_ADD, out=SK), L.OK),
    (dict(op=L.OP_BIAS_ADD, mode=2, skip_rows=2), L.ERR_MODE),
    (dict(op=L.OP_SIMPLIFIED, mode=2, skip_rows=2), L.ERR_MODE),   # grouped reuse is BiasSoftmax's
    # BiasSoftmax: input = data, skip = bias rows; gamma/beta/bias/residual/eps ignored
    (dict(op=L.OP_BIAS_SOFTMAX), L.OK),
    (dict(op=L.OP_BIAS_SOFTMAX, gamma=None, beta=None, bias=None, res=None, eps=-1.0), L.OK),
    (dict(op=L.OP_BIAS_SOFTMAX, res=IN + 4, bias=OUT), L.OK),
    (dict(op=L.OP_BIAS_SOFTMAX, mode=1, skip_rows=2), L.OK),
    (dict(op=L.OP_BIAS_SOFTMAX, mode=2, skip_rows=2), L.OK),
    (dict(op=L.OP_BIAS_SOFTMAX, mode=2, skip_rows=4), L.OK),
    (dict(op=L.OP_BIAS_SOFTMAX, mode=2, skip_rows=3), L.ERR_SHAPE),
    (dict(op=L.OP_BIAS_SOFTMAX, mode=2, skip_rows=0), L.ERR_SHAPE),
    (dict(op=L.OP_BIAS_SOFTMAX, mode=3, skip_rows=2), L.ERR_MODE),
    (dict(op=L.OP_BIAS_SOFTMAX, skip=None), L.ERR_NULL),
    (dict(op=L.OP_BIAS_SOFTMAX, out=IN), L.OK),
    (dict(op=L.OP_BIAS_SOFTMAX, out=SK), L.OK),                  # exact bias: read row by row
    (dict(op=L.OP_BIAS_SOFTMAX, out=SK, mode=2, skip_rows=2), L.ERR_ALIAS),
    (dict(op=L.OP_BIAS_SOFTMAX, out=IN + 16), L.ERR_ALIAS),
])
def test_validate_operations(kw, status):
    assert V(**kw) == status


def S(data=IN, bias=SK, out=OUT, batch=4, block=8, bias_rows=2, inner=0, dtype=0):
    return L.load().skipln_bias_softmax(data, bias, out, batch, block, bias_rows, inner, dtype, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    # `biasContract`: empty data with an empty bias is a no-op (no HIP call)
    (dict(batch=0, bias_rows=0), L.OK),
    (dict(block=0, bias_rows=3), L.OK),
    (dict(batch=0, block=0, bias_rows=0, data=None, bias=None, out=None), L.OK),
    (dict(batch=0, bias_rows=0, dtype=7), L.ERR_DTYPE),
    (dict(batch=0, bias_rows=1), L.ERR_SHAPE),    # bias rows but no data rows
    (dict(bias_rows=0), L.ERR_SHAPE),
    (dict(bias_rows=3), L.ERR_SHAPE),             # 4 rows not a multiple of 3
    (dict(bias_rows=8), L.ERR_SHAPE),             # more bias rows than data rows
    (dict(batch=-4), L.ERR_SHAPE),
    (dict(block=-8), L.ERR_SHAPE),
    (dict(bias_rows=-2), L.ERR_SHAPE),
    (dict(block=2 ** 31), L.ERR_SHAPE),
    (dict(dtype=2), L.ERR_DTYPE),
    (dict(data=None), L.ERR_NULL),
    (dict(bias=None, inner=1), L.ERR_NULL),
    (dict(out=None), L.ERR_NULL),
    (dict(out=SK), L.ERR_ALIAS),                  # broadcast bias is read by several rows
    (dict(out=SK, inner=1), L.ERR_ALIAS),
    (dict(out=IN + 4), L.ERR_ALIAS),
])
def test_bias_softmax_argument_checks(kw, status):
    """Every status reached here returns before any HIP call."""
    assert S(**kw) == status


def test_validate_rows_zero_is_a_noop_even_with_null_pointers():
    assert V(rows=0, input=None, skip=None, gamma=None, out=None) == L.OK


def test_validate_allows_exact_aliasing():
    assert V(out=IN) == L.OK                 # in place over input
    assert V(res=IN, out=SK) == L.OK         # residual over input, output over exact skip
    assert V(out=IN, res=None) == L.OK
    assert V(beta=None, out=BE) == L.OK      # an absent beta occupies no memory


CUS = 256  # MI355X compute units, given explicitly: select then makes no HIP call


def SEL(op, h, dt, mode=L.SKIP_EXACT, al=1, v=L.VARIANT_AUTO, ws=0, rows=-1, cus=CUS):
    return L.load_tune().skipln_tune_select(op, rows, h, dt, mode, al, v, ws, cus)


def test_select_kernels():
    lib = L.load_tune()
    sel = lambda h, dt, al=1, v=0, mode=L.SKIP_EXACT, op=L.OP_LAYER_NORM: SEL(op, h, dt, mode, al, v)
    name = lambda kid: L.kernel_name(kid)
    assert name(sel(768, 0)) == "rowtile_f32_g192_c1_b192"
    assert name(sel(1024, 1)) == "rowtile_f16_g64_c2"                 # one wavefront per row
    assert name(sel(1024, 1, op=L.OP_BIAS_ADD)) == "biasadd_rowtile_f16_g128_c1"
    assert name(sel(768, 0, mode=L.SKIP_BROADCAST)) == "rowtile_f32_g192_c1_b192"
    assert name(sel(768, 0, op=L.OP_BIAS_ADD)) == "biasadd_rowtile_f32_g192_c1_b192"
    assert name(sel(4096, 0)) == "rowtile_f32_g256_c4"
    assert name(sel(4096, 0, mode=L.SKIP_BROADCAST)) == "rowtile_f32_g256_c4"
    assert name(sel(8192, 1)) == "rowtile_f16_g256_c4"
    assert name(sel(64, 0)) == "rowtile_f32_g16_c1"
    # not a multiple of a 16-byte chunk with 16-byte aligned tensors and an
    # exact skip: span row tiles for BiasSoftmax rows touching 8 to 2048
    # chunks and BiasAdd rows touching 64 to 2048; the normalizations,
    # misaligned tensors, broadcast forms and other lengths: element-wise row
    # tiles; too long for every family: generic
    assert name(sel(1001, 0)) == "rowelem_f32_g128_c8"
    assert name(sel(77, 1)) == "rowelem_f16_g32_c4"
    assert name(sel(3, 1)) == "rowelem_f16_g4_c1"
    assert name(sel(1500, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_span_f16_g64_c3"     # 189 chunks touched
    assert name(sel(2039, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_span_f16_g64_c4"     # 256
    assert name(sel(2047, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_span_f16_g128_c3"    # 257
    assert name(sel(49, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_span_f16_g8_c2"      # 8 chunks touched
    assert name(sel(47, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_rowelem_f16_g16_c4"  # 7
    assert name(sel(2039, 1)) == "rowelem_f16_g256_c8"
    assert name(sel(16366, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_span_f16_g512_c4"    # 2047 chunks touched
    assert name(sel(16378, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_rowelem_f16_g1024_c16"
    assert name(sel(1500, 1, op=L.OP_BIAS_SOFTMAX, mode=L.SKIP_BROADCAST)) == "softmax_rowelem_f16_g256_c8"
    assert name(sel(1001, 0, mode=L.SKIP_BROADCAST)) == "rowelem_f32_g128_c8"
    assert name(sel(1001, 0, al=0)) == "rowelem_f32_g128_c8"
    assert name(sel(1024, 0, al=0)) == "rowelem_f32_g128_c8"
    assert name(sel(77, 1, al=0)) == "rowelem_f16_g32_c4"
    assert name(sel(3, 1, al=0)) == "rowelem_f16_g4_c1"
    assert name(sel(16384, 1, al=0)) == "rowelem_f16_g1024_c16"
    assert name(sel(16385, 1, al=0)) == "generic_f16"
    assert sel(16385, 1, v=L.VARIANT_ELEMENT) == -L.ERR_UNSUPPORTED
    assert name(sel(1000, 0, v=L.VARIANT_ELEMENT)) == "rowelem_f32_g128_c8"
    assert sel(1000, 0, v=L.VARIANT_ELEMENT_GEOMETRY + 0) == -L.ERR_UNSUPPORTED   # 4 elements
    assert name(sel(4, 0, v=L.VARIANT_ELEMENT_GEOMETRY + 0)) == "rowelem_f32_g4_c1"
    ns = lib.skipln_tune_span_geometries()
    assert ns == 12
    assert sel(4, 0, v=L.VARIANT_SPAN_GEOMETRY + ns) == -L.ERR_VARIANT
    assert sel(4, 0, al=0, v=L.VARIANT_SPAN) == -L.ERR_UNSUPPORTED              # needs 16-byte aligned tensors
    assert sel(4001, 0, v=L.VARIANT_SPAN_GEOMETRY + 0) == -L.ERR_UNSUPPORTED    # too long for 8 x 2
    assert name(sel(1024, 0, v=L.VARIANT_SPAN)) == "span_f32_g128_c3"           # any length when forced
    for g in range(ns):
        assert name(sel(5, 1, v=L.VARIANT_SPAN_GEOMETRY + g)).startswith("span_f16_g")
    ne = lib.skipln_tune_element_geometries()
    assert ne == 13
    assert sel(4, 0, v=L.VARIANT_ELEMENT_GEOMETRY + ne) == -L.ERR_VARIANT
    for g in range(ne):
        assert name(sel(4, 0, v=L.VARIANT_ELEMENT_GEOMETRY + g)).startswith("rowelem_f32_g")
    assert name(sel(20000, 0)) == "ldsrow_f32"
    assert name(sel(50000, 0)) == "regrow_f32"                      # held in registers
    assert name(sel(8, 1, v=1)) == "generic_f16"
    assert sel(1001, 0, v=L.VARIANT_ROWTILE) == -L.ERR_UNSUPPORTED
    assert name(sel(64, 0, v=L.VARIANT_MULTIWAVE)).startswith("rowtile_f32_g128")
    ng = lib.skipln_tune_rowtile_geometries()
    assert ng == 23
    for g in range(ng):
        kid = sel(16, 0, v=L.VARIANT_GEOMETRY + g)   # 4 chunks: every geometry holds them
        assert kid >= 0 and name(kid).startswith("rowtile_f32_g")
    assert sel(16384, 0, v=L.VARIANT_GEOMETRY + 0) == -L.ERR_UNSUPPORTED
    assert sel(64, 0, v=L.VARIANT_GEOMETRY + ng) == -L.ERR_VARIANT
    assert sel(64, 0, v=17) == -L.ERR_VARIANT
    assert sel(64, 5) == -L.ERR_DTYPE
    assert sel(0, 0) == -L.ERR_SHAPE
    assert sel(64, 0, mode=3) == -L.ERR_MODE
    assert sel(64, 0, op=7) == -L.ERR_OP
    assert name(sel(768, 0, op=L.OP_SIMPLIFIED)) == "rms_rowtile_f32_g192_c1_b192"
    assert name(sel(4096, 1, op=L.OP_BIAS_ADD)) == "biasadd_rowtile_f16_g256_c2"
    assert name(sel(1001, 1, op=L.OP_BIAS_ADD)) == "biasadd_span_f16_g64_c2"
    assert name(sel(497, 1, op=L.OP_BIAS_ADD)) == "biasadd_span_f16_g32_c2"      # 64 chunks touched
    assert name(sel(495, 1, op=L.OP_BIAS_ADD)).startswith("biasadd_rowelem_f16")  # 63
    assert name(sel(1001, 1, al=0, op=L.OP_BIAS_ADD)) == "biasadd_rowelem_f16_g128_c8"
    # long rows: LDS-staged up to 163584 bytes of binary32 sums, then held
    # in registers up to 65536 values, then generic
    assert name(sel(8192, 0)) == "rowtile_f32_g1024_c3"     # float32 layer norm, 1537-2048 chunks of whole lines
    assert name(sel(8184, 0)) == "rowtile_f32_g512_c4"      # rows ending inside a line
    assert name(sel(8192, 0, op=L.OP_SIMPLIFIED)) == "rms_rowtile_f32_g512_c4"
    assert name(sel(8196, 0)) == "ldsrow_f32"
    assert name(sel(40896, 0)) == "ldsrow_f32"
    assert name(sel(40900, 0)) == "regrow_f32"
    assert name(sel(65536, 1, op=L.OP_SIMPLIFIED)) == "rms_regrow_f16"
    assert name(sel(65540, 0)) == "generic_f32"
    assert name(sel(16392, 1, op=L.OP_SIMPLIFIED)) == "rms_ldsrow_f16"
    assert name(sel(16392, 1, op=L.OP_BIAS_ADD)) == "biasadd_rowtile_f16_g1024_c3"
    assert name(sel(64, 0, v=L.VARIANT_LDSROW)) == "ldsrow_f32"
    assert sel(64, 0, v=L.VARIANT_LDSROW, op=L.OP_BIAS_ADD) == -L.ERR_UNSUPPORTED
    # tiny rows pack 64 or 32 rows into a 256-lane block
    assert name(sel(16, 0)) == "rowtile_f32_g4_c1"
    assert name(sel(32, 1)) == "rowtile_f16_g4_c1"
    assert name(sel(32, 0)) == "rowtile_f32_g8_c1"
    # BiasSoftmax: every skip form, the same families
    assert name(sel(512, 1, op=L.OP_BIAS_SOFTMAX, mode=L.SKIP_BROADCAST_INNER)) == "softmax_rowtile_f16_g32_c2"
    assert name(sel(8, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_rowtile_f16_g4_c1"
    assert name(sel(8, 0, op=L.OP_BIAS_SOFTMAX, mode=L.SKIP_BROADCAST)) == "softmax_rowtile_f32_g4_c1"
    assert name(sel(4096, 1, op=L.OP_BIAS_SOFTMAX)) == "softmax_rowtile_f16_g128_c4"
    assert name(sel(20000, 0, op=L.OP_BIAS_SOFTMAX)) == "softmax_ldsrow_f32"
    assert name(sel(7, 0, op=L.OP_BIAS_SOFTMAX)) == "softmax_rowelem_f32_g4_c2"
    assert name(sel(25, 0, op=L.OP_BIAS_SOFTMAX)) == "softmax_span_f32_g8_c2"
    assert name(sel(7, 0, al=0, op=L.OP_BIAS_SOFTMAX)) == "softmax_rowelem_f32_g4_c2"
    assert name(sel(64, 1, op=L.OP_BIAS_SOFTMAX, v=L.VARIANT_LDSROW)) == "softmax_ldsrow_f16"
    assert sel(64, 0, mode=L.SKIP_BROADCAST_INNER) == -L.ERR_MODE
    assert sel(66, 0, v=L.VARIANT_LDSROW) == -L.ERR_UNSUPPORTED
    assert L.kernel_name(-1) == "unknown" and L.kernel_name(10 ** 6) == "unknown"


def test_every_geometry_is_an_automatic_choice():
    """Each row-tile, element-wise and span geometry is what the automatic
    choice takes for some operation, type, skip form and row length."""
    lib = L.load_tune()
    used, used_elem = set(), set()
    for op in (L.OP_LAYER_NORM, L.OP_BIAS_ADD, L.OP_BIAS_SOFTMAX):
        for dt, v in ((0, 4), (1, 8)):
            for mode in (L.SKIP_EXACT, L.SKIP_BROADCAST):
                if op == L.OP_BIAS_ADD and mode != L.SKIP_EXACT:
                    continue
                for hv in range(1, 4097):
                    used.add(L.kernel_name(SEL(op, hv * v, dt, mode)).split("_", 1)[-1].replace("rowtile_", "")
                             .split("_", 1)[-1])
            for h in range(1, 16385):
                n = L.kernel_name(SEL(op, h, dt, al=0))
                if "rowelem_" in n:
                    used_elem.add(n.split("rowelem_")[1].split("_", 1)[1])
    names = {L.kernel_name(SEL(L.OP_LAYER_NORM, 4, 0, v=L.VARIANT_GEOMETRY + g)).split("rowtile_f32_")[1]
             for g in range(lib.skipln_tune_rowtile_geometries())}
    assert names <= used, f"geometries no automatic choice takes: {names - used}"
    elems = {L.kernel_name(SEL(L.OP_LAYER_NORM, 1, 0, al=0, v=L.VARIANT_ELEMENT_GEOMETRY + g)).split("rowelem_f32_")[1]
             for g in range(lib.skipln_tune_element_geometries())}
    assert elems <= used_elem, f"element geometries no automatic choice takes: {elems - used_elem}"
    used_span = {L.kernel_name(SEL(op, h, dt)).split("span_")[1].split("_", 1)[1]
                 for op in (L.OP_BIAS_ADD, L.OP_BIAS_SOFTMAX) for dt in (0, 1) for h in range(1, 16385, 3)
                 if "span_" in L.kernel_name(SEL(op, h, dt))}
    spans = {L.kernel_name(SEL(L.OP_LAYER_NORM, 1, 0, v=L.VARIANT_SPAN_GEOMETRY + g)).split("span_f32_")[1]
             for g in range(lib.skipln_tune_span_geometries())}
    assert spans <= used_span, f"span geometries no automatic choice takes: {spans - used_span}"


def test_auto_choice_holds_every_hidden_size():
    """The automatic choice exists for every chunked hidden size up to the
    row-tile limit, holds the row, and is monotone in capacity."""
    lib = L.load_tune()
    for dt, v in ((0, 4), (1, 8)):
        for mode in (L.SKIP_EXACT, L.SKIP_BROADCAST):
            for hv in range(1, 2049):
                kid = SEL(L.OP_LAYER_NORM, hv * v, dt, mode)
                assert kid >= 0 and L.kernel_name(kid).startswith("rowtile_"), (dt, mode, hv)
                n = L.kernel_name(kid)
                g = int(n.split("_g")[1].split("_")[0])
                c = int(n.split("_c")[1].split("_")[0])
                assert g * c >= hv
            for hv in range(2049, 4097):
                kid = SEL(L.OP_BIAS_ADD, hv * v, dt)
                n = L.kernel_name(kid)
                assert n.startswith("biasadd_rowtile_"), (dt, hv, n)
            assert L.kernel_name(SEL(L.OP_BIAS_ADD, 4097 * v, dt)).startswith("biasadd_generic_")
        for mode in (L.SKIP_EXACT, L.SKIP_BROADCAST, L.SKIP_BROADCAST_INNER):
            for hv in range(1, 2049):
                n = L.kernel_name(SEL(L.OP_BIAS_SOFTMAX, hv * v, dt, mode))
                assert n.startswith("softmax_rowtile_"), (dt, mode, hv, n)
                g = int(n.split("_g")[1].split("_")[0])
                c = int(n.split("_c")[1].split("_")[0])
                assert g * c >= hv and (g * c < 2 * hv or g * c == 4), (hv, n)


def test_no_cpu_fallback_in_product_path():
    """The package never imports the oracle and has no CPU path."""
    pkg = os.path.join(ROOT, "transformer_residual_add_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from\s+oracle|import\s+oracle)|liboracle|skipln_oracle", text, re.M), \
                    f"{f} reaches into the oracle"


# ------------------------------------------------------------- workspace --

def test_workspace_sizes_and_split_selection():
    lib, tune = L.load(), L.load_tune()
    wb = lambda op, rows, h, dt, mode=L.SKIP_EXACT, srows=0: lib.skipln_workspace_bytes(op, rows, h, dt, mode, srows)
    wbv = lambda op, rows, h, dt, mode=L.SKIP_EXACT, srows=0, v=L.VARIANT_AUTO: \
        tune.skipln_tune_workspace_bytes(op, rows, h, dt, mode, srows, v)
    name = lambda op, h, dt, v=L.VARIANT_AUTO, mode=L.SKIP_EXACT, ws=0, rows=-1, cus=CUS: \
        L.kernel_name(SEL(op, h, dt, mode, 1, v, ws, rows, cus))
    # one float4 partial per slice of a batch of rows; a batch streams at most
    # 128 MiB of inputs (x, and skip when it is not broadcast)
    ws = lambda rows, slices: rows * slices * 16
    assert wb(L.OP_LAYER_NORM, 64, 131072, L.F32) == ws(64, 32)
    assert wbv(L.OP_LAYER_NORM, 1000, 65536, L.F32, v=L.VARIANT_SPLITROW) == ws(256, 16)
    assert wbv(L.OP_LAYER_NORM, 1000, 65536, L.F32, L.SKIP_BROADCAST, 8, L.VARIANT_SPLITROW) == ws(512, 16)
    # the operator library's size does not depend on the device: whatever the
    # row count, a call that may split its rows gets the split-row size
    for rows in (255, 256, 1000):
        assert wb(L.OP_LAYER_NORM, rows, 131072, L.F32) == \
            wbv(L.OP_LAYER_NORM, rows, 131072, L.F32, v=L.VARIANT_SPLITROW) > 0
    assert wb(L.OP_LAYER_NORM, 1000, 131072, L.F32, L.SKIP_BROADCAST, 8) == ws(256, 32)
    assert wb(L.OP_LAYER_NORM, 1000, 131072, L.F16) == ws(256, 16)
    # rows held in registers need none
    assert wb(L.OP_LAYER_NORM, 64, 65536, L.F32) == 0
    assert wb(L.OP_LAYER_NORM, 1000, 65536, L.F16) == 0
    assert wb(L.OP_SIMPLIFIED, 255, 262144, L.F32) == ws(64, 64)
    assert wb(L.OP_BIAS_SOFTMAX, 1024, 163848, L.F16) > 0
    assert wb(L.OP_LAYER_NORM, 201, 65540, L.F32) == ws(201, 17)
    assert wb(L.OP_LAYER_NORM, 0, 65536, L.F32) == 0
    assert wb(L.OP_LAYER_NORM, 64, 4096, L.F32) == 0                       # row tiles need none
    assert wb(L.OP_LAYER_NORM, 64, 20000, L.F32) == 0                      # LDS-staged
    assert wbv(L.OP_LAYER_NORM, 64, 4096, L.F32, v=L.VARIANT_SPLITROW) == ws(64, 1)
    assert wbv(L.OP_BIAS_ADD, 64, 65536, L.F32, v=L.VARIANT_SPLITROW) == -L.ERR_UNSUPPORTED
    assert wbv(L.OP_LAYER_NORM, 64, 4096, L.F32, v=L.VARIANT_GENERIC) == 0
    assert wb(L.OP_LAYER_NORM, 64, 65536, 9) == -L.ERR_DTYPE
    assert wb(L.OP_LAYER_NORM, 64, 65536, L.F32, L.SKIP_BROADCAST, 3) == -L.ERR_SHAPE
    assert wb(7, 64, 65536, L.F32) == -L.ERR_OP
    assert wb(L.OP_BIAS_SOFTMAX, 64, 128256, L.F16, L.SKIP_BROADCAST_INNER, 4) == 0     # held in registers
    assert wbv(L.OP_BIAS_SOFTMAX, 64, 128256, L.F16, L.SKIP_BROADCAST_INNER, 4, L.VARIANT_SPLITROW) == ws(64, 16)
    assert wb(L.OP_BIAS_SOFTMAX, 64, 163848, L.F16) == ws(64, 21)                     # beyond the registers
    # the automatic choice: rows up to 65536 values held in registers, with
    # or without a workspace, whatever the row count ...
    for ws_ in (0, 1):
        for rows in (-1, 1, 10 ** 6):
            assert name(L.OP_LAYER_NORM, 65536, L.F32, ws=ws_, rows=rows) == "regrow_f32"
            assert name(L.OP_SIMPLIFIED, 65536, L.F16, ws=ws_, rows=rows) == "rms_regrow_f16"
    # ... longer rows split only where a workspace is at hand, and with fewer
    # rows than the device has compute units: from one row per CU, RMS runs
    # generic
    assert name(L.OP_LAYER_NORM, 131072, L.F32) == "generic_f32"
    assert name(L.OP_LAYER_NORM, 131072, L.F32, ws=1) == "splitrow_f32"
    for cus in (256, 80):
        assert name(L.OP_SIMPLIFIED, 262144, L.F32, ws=1, rows=cus, cus=cus) == "rms_generic_f32"
        assert name(L.OP_SIMPLIFIED, 262144, L.F32, ws=1, rows=cus - 1, cus=cus) == "rms_splitrow_f32"
    assert name(L.OP_LAYER_NORM, 65540, L.F32, ws=1, rows=1000) == "splitrow_f32"       # beyond 65536
    assert name(L.OP_LAYER_NORM, 131072, L.F16, ws=1, rows=1000) == "splitrow_f16"      # float16 keeps it
    assert name(L.OP_BIAS_SOFTMAX, 128256, L.F16, ws=1) == "softmax_regrow_f16"
    assert name(L.OP_BIAS_SOFTMAX, 163848, L.F16, ws=1) == "softmax_splitrow_f16"
    assert name(L.OP_LAYER_NORM, 20000, L.F32, ws=1) == "ldsrow_f32"
    assert name(L.OP_LAYER_NORM, 4096, L.F32, ws=1) == "rowtile_f32_g256_c4"
    assert name(L.OP_LAYER_NORM, 64 * 4096, L.F32, ws=1) == "splitrow_f32"        # 64 slices
    assert name(L.OP_LAYER_NORM, 64 * 4096 + 4, L.F32, ws=1) == "generic_f32"     # 65 slices
    assert name(L.OP_BIAS_ADD, 65536, L.F32, ws=1) == "biasadd_generic_f32"
    assert name(L.OP_LAYER_NORM, 64, L.F32, v=L.VARIANT_SPLITROW) == "splitrow_f32"
    assert SEL(L.OP_BIAS_ADD, 64, L.F32, v=L.VARIANT_SPLITROW) == -L.ERR_UNSUPPORTED
    assert SEL(L.OP_LAYER_NORM, 66, L.F32, v=L.VARIANT_SPLITROW) == -L.ERR_UNSUPPORTED


def test_register_resident_softmax_selection():
    """BiasSoftmax rows beyond the LDS capacity and up to 20 chunks per lane
    of a 1024-lane block are held in registers, with or without a
    workspace; the family takes only 16-byte chunks of BiasSoftmax."""
    name = lambda h, dt, v=L.VARIANT_AUTO, mode=L.SKIP_EXACT, op=L.OP_BIAS_SOFTMAX, al=1: \
        L.kernel_name(SEL(op, h, dt, mode, al, v))
    name_ws = lambda h, dt, mode=L.SKIP_EXACT: L.kernel_name(SEL(L.OP_BIAS_SOFTMAX, h, dt, mode, ws=1))
    for mode in (L.SKIP_EXACT, L.SKIP_BROADCAST, L.SKIP_BROADCAST_INNER):
        assert name(40896, L.F32, mode=mode) == "softmax_ldsrow_f32"
        assert name(40900, L.F32, mode=mode) == "softmax_regrow_f32"
        assert name(65536, L.F32, mode=mode) == "softmax_regrow_f32"
        assert name(81920, L.F32, mode=mode) == "softmax_regrow_f32"
        assert name(81924, L.F32, mode=mode) == "softmax_generic_f32"
        assert name_ws(81924, L.F32, mode) == "softmax_splitrow_f32"
        assert name(40960, L.F16, mode=mode) == "softmax_regrow_f16"
        assert name(131072, L.F16, mode=mode) == "softmax_regrow_f16"
        assert name_ws(131072, L.F16, mode) == "softmax_regrow_f16"
        assert name(163840, L.F16, mode=mode) == "softmax_regrow_f16"
        assert name(163848, L.F16, mode=mode) == "softmax_generic_f16"
    # forced: any row of whole chunks up to the capacity
    assert name(8, L.F32, v=L.VARIANT_REGROW) == "softmax_regrow_f32"
    assert name(4096, L.F16, v=L.VARIANT_REGROW) == "softmax_regrow_f16"
    unsupported = -L.ERR_UNSUPPORTED
    assert SEL(L.OP_BIAS_SOFTMAX, 81924, L.F32, v=L.VARIANT_REGROW) == unsupported
    assert SEL(L.OP_BIAS_SOFTMAX, 77, L.F32, v=L.VARIANT_REGROW) == unsupported    # not chunks
    assert SEL(L.OP_BIAS_SOFTMAX, 4096, L.F32, al=0, v=L.VARIANT_REGROW) == unsupported  # misaligned
    assert SEL(L.OP_BIAS_ADD, 65536, L.F16, v=L.VARIANT_REGROW) == unsupported
    # the normalizations' register-resident rows (forced): 32776-65536
    # float16, 36868-65536 float32 values
    assert name(65536, L.F16, v=L.VARIANT_REGROW, op=L.OP_LAYER_NORM) == "regrow_f16"
    assert name(32776, L.F16, v=L.VARIANT_REGROW, op=L.OP_SIMPLIFIED) == "rms_regrow_f16"
    assert name(36868, L.F32, v=L.VARIANT_REGROW, op=L.OP_LAYER_NORM) == "regrow_f32"
    for op in (L.OP_LAYER_NORM, L.OP_SIMPLIFIED):
        assert SEL(op, 32768, L.F16, v=L.VARIANT_REGROW) == unsupported
        assert SEL(op, 36864, L.F32, v=L.VARIANT_REGROW) == unsupported
        assert SEL(op, 65544, L.F16, v=L.VARIANT_REGROW) == unsupported
        assert SEL(op, 65540, L.F32, v=L.VARIANT_REGROW) == unsupported
    # misaligned long rows take the generic kernel
    assert name(65536, L.F16, al=0) == "softmax_generic_f16"


def FW(ws, nbytes, hidden=131072, variant=L.VARIANT_AUTO, op=L.OP_LAYER_NORM, res=RES):
    """skipln_forward_ws (automatic choice) or the tuning library's forced
    family, on fake pointers: every status here returns before any HIP call."""
    args = (IN, SK, 0, 0, GA, BE, BI, OUT, res, 2, hidden, 1e-5, L.F32)
    if variant == L.VARIANT_AUTO:
        return L.load().skipln_forward_ws(op, *args, ws, nbytes, None)
    return L.load_tune().skipln_tune_forward(op, *args, variant, ws, nbytes, None)


WS = 0x10000000  # beyond every fake tensor (2 rows of 131072 float32 = 1 MiB each)


def test_forward_ws_workspace_checks():
    need = L.load().skipln_workspace_bytes(L.OP_LAYER_NORM, 2, 131072, L.F32, 0, 0)
    assert need == 2 * 32 * 16
    assert FW(None, 0) == L.ERR_WORKSPACE
    assert FW(WS, need - 1) == L.ERR_WORKSPACE
    assert FW(WS + 8, need) == L.ERR_WORKSPACE          # not 16-byte aligned
    assert FW(WS, -1) == L.ERR_WORKSPACE
    assert FW(IN, need) == L.ERR_ALIAS                  # overlaps the input
    assert FW(OUT + 64, need) == L.ERR_ALIAS
    assert FW(WS, need, variant=L.VARIANT_LDSROW) == L.ERR_UNSUPPORTED
    assert FW(None, 0, hidden=64, variant=L.VARIANT_SPLITROW) == L.ERR_WORKSPACE
    assert FW(WS, need, op=L.OP_BIAS_ADD, variant=L.VARIANT_SPLITROW) == L.ERR_UNSUPPORTED
    assert FW(WS, need, variant=99) == L.ERR_VARIANT
    # a residual over the input cannot take the split-row kernels (they read x twice)
    assert FW(WS, need, variant=L.VARIANT_SPLITROW, res=IN) == L.ERR_UNSUPPORTED
    assert L.load().skipln_forward_ws(9, IN, SK, 0, 0, GA, BE, BI, OUT, RES, 4, 8, 1e-5, L.F32, WS, need, None) \
        == L.ERR_OP


def test_forward_config_argument_checks():
    """skipln_tune_forward_config rejects these before any HIP call."""
    cfg = lambda geom=0, tpb=1, tiling=0, store=L.STORE_AUTO: L.load_tune().skipln_tune_forward_config(
        L.OP_LAYER_NORM, IN, SK, 0, 0, GA, BE, BI, OUT, RES, 4, 64, 1e-5, L.F32, geom, tpb, tiling, store, None)
    assert cfg(tpb=-1) == L.ERR_SHAPE
    assert cfg(tiling=3) == L.ERR_VARIANT
    assert cfg(store=2) == L.ERR_VARIANT and cfg(store=-2) == L.ERR_VARIANT
    assert cfg(geom=-2) == L.ERR_VARIANT
    assert cfg(geom=L.load_tune().skipln_tune_rowtile_geometries()) == L.ERR_VARIANT
    assert cfg(geom=L.VARIANT_ELEMENT_GEOMETRY + L.load_tune().skipln_tune_element_geometries()) == L.ERR_VARIANT


def test_large_launches_take_1024_lane_row_tiles():
    """Normalization rows of 2049-3072 chunks (float16: 2689-3072; float32 up
    to 4096) of whole 128-byte lines leave the LDS-staged kernel for 1024-lane
    row tiles once
    input, skip and output each span 512 MiB; broadcast skips, BiasSoftmax and
    other lengths do not."""
    sel = lambda h, dt, rows, op=L.OP_LAYER_NORM, mode=L.SKIP_EXACT: L.kernel_name(L.load_tune().skipln_tune_select(
        op, rows, h, dt, mode, 1, L.VARIANT_AUTO, 0, 256))
    big = lambda h, dt: -(-(512 << 20) // (h * (4 if dt == L.F32 else 2)))
    for h, dt in ((8224, L.F32), (10240, L.F32), (12288, L.F32), (21568, L.F16), (24576, L.F16)):
        n = big(h, dt)
        for op, prefix in ((L.OP_LAYER_NORM, ""), (L.OP_SIMPLIFIED, "rms_")):
            assert sel(h, dt, n, op) == f"{prefix}rowtile_{'f32' if dt == L.F32 else 'f16'}_g1024_c3"
            assert sel(h, dt, n - 1, op).startswith(f"{prefix}ldsrow_")
        assert sel(h, dt, n, mode=L.SKIP_BROADCAST).startswith("ldsrow_")
        assert sel(h, dt, n, L.OP_BIAS_SOFTMAX).startswith("softmax_")
    # too short, too long, or rows that end inside a 128-byte line
    for h, dt in ((21504, L.F16), (24640, L.F16), (8196, L.F32), (22600, L.F16)):
        assert "g1024_c3" not in sel(h, dt, big(h, dt))
    # float32 rows of 3073-4096 chunks: 1024 x 4 tiles; float16 rows of that
    # length stay on the LDS-staged kernel
    for h in (12416, 14336, 16384):
        for op, prefix in ((L.OP_LAYER_NORM, ""), (L.OP_SIMPLIFIED, "rms_")):
            assert sel(h, L.F32, big(h, L.F32), op) == f"{prefix}rowtile_f32_g1024_c4"
            assert sel(h, L.F32, big(h, L.F32) - 1, op) == f"{prefix}ldsrow_f32"
    assert sel(16416, L.F32, big(16416, L.F32)) == "ldsrow_f32"
    assert sel(32768, L.F16, big(32768, L.F16)) == "ldsrow_f16"
    # float16 RMS from 2304 chunks
    assert sel(18432, L.F16, big(18432, L.F16), L.OP_SIMPLIFIED) == "rms_rowtile_f16_g1024_c3"
    assert sel(18368, L.F16, big(18368, L.F16), L.OP_SIMPLIFIED) == "rms_ldsrow_f16"
    assert sel(18432, L.F16, big(18432, L.F16)) == "ldsrow_f16"


def test_row_count_dependent_choices():
    """The normalizations' row tiles that depend on the launch's rows: one
    wavefront per row for 161-256 chunks from 16384 rows (below the
    single-tile size), 128 x 4 tiles for 257-512 chunks except in single-tile
    launches (256 x 2)."""
    sel = lambda h, dt, rows, op=L.OP_LAYER_NORM, mode=L.SKIP_EXACT: L.kernel_name(L.load_tune().skipln_tune_select(
        op, rows, h, dt, mode, 1, L.VARIANT_AUTO, 0, 256))
    assert sel(2048, L.F16, 16384) == "rowtile_f16_g64_c4"
    assert sel(2048, L.F16, 16383) == "rowtile_f16_g256_c1"
    assert sel(1288, L.F16, 32768) == "rowtile_f16_g64_c4"                 # 161 chunks
    assert sel(1280, L.F16, 32768) == "rowtile_f16_g192_c1_b192"           # 160
    assert sel(768, L.F32, 131072, L.OP_SIMPLIFIED) == "rms_rowtile_f32_g64_c4"
    assert sel(768, L.F32, 1024) == "rowtile_f32_g192_c1_b192"            # BERT-base
    assert sel(2048, L.F16, 131072) == "rowtile_f16_g256_c1"               # single-tile launch
    assert sel(1536, L.F16, 262144) == "rowtile_f16_g64_c4"                # ... but not at 161-192 chunks
    assert sel(2048, L.F16, 32768, mode=L.SKIP_BROADCAST) == "rowtile_f16_g64_c4"
    assert sel(2048, L.F16, 32768, L.OP_BIAS_ADD) == "biasadd_rowtile_f16_g256_c1"
    assert sel(4096, L.F16, 32768) == "rowtile_f16_g128_c4"
    assert sel(4096, L.F16, 65536) == "rowtile_f16_g256_c2"                # single-tile launch
    assert sel(4096, L.F16, 32768, mode=L.SKIP_BROADCAST) == "rowtile_f16_g128_c4"


def test_forward_form_argument_checks():
    """skipln_tune_forward_form rejects these before any HIP call."""
    frm = lambda geom=0, form=1, cap=0, store=L.STORE_AUTO: L.load_tune().skipln_tune_forward_form(
        L.OP_LAYER_NORM, IN, SK, 0, 0, GA, BE, BI, OUT, RES, 4, 64, 1e-5, L.F32, geom, form, cap, store, None)
    assert frm(form=2) == L.ERR_VARIANT and frm(form=-1) == L.ERR_VARIANT
    assert frm(cap=-2) == L.ERR_VARIANT
    assert frm(store=2) == L.ERR_VARIANT
    assert frm(geom=-2) == L.ERR_VARIANT
    assert frm(geom=L.load_tune().skipln_tune_rowtile_geometries()) == L.ERR_VARIANT
    # the argument checks of the operator itself still come first for the rest
    assert frm(geom=L.VARIANT_ELEMENT_GEOMETRY) == L.ERR_VARIANT


def test_blocks_per_cu_argument_checks():
    """skipln_tune_blocks_per_cu rejects these before any HIP call."""
    bpc = lambda op=L.OP_LAYER_NORM, dt=L.F16, geom=0, form=1, cap=0: L.load_tune().skipln_tune_blocks_per_cu(
        op, dt, geom, form, cap)
    assert bpc(op=9) == -L.ERR_OP
    assert bpc(dt=5) == -L.ERR_DTYPE
    assert bpc(geom=-1) == -L.ERR_VARIANT
    assert bpc(geom=L.load_tune().skipln_tune_rowtile_geometries()) == -L.ERR_VARIANT
    assert bpc(form=2) == -L.ERR_VARIANT and bpc(form=-1) == -L.ERR_VARIANT
    assert bpc(cap=-2) == -L.ERR_VARIANT


def test_stream_probe_argument_checks():
    """skipln_tune_stream returns these statuses before any HIP call."""
    st = lambda s0=IN, s1=None, d0=OUT, d1=None, n=4096, b=256, u=4, g=1: L.load_tune().skipln_tune_stream(s0, s1, d0,
                                                                                                 d1, n, b,
                                                                                                 u, g, 0, None)
    assert st(s0=None, d0=None) == L.ERR_NULL
    assert st(s0=None, s1=SK) == L.ERR_NULL
    assert st(d0=None, d1=RES) == L.ERR_NULL
    assert st(n=-16) == L.ERR_SHAPE
    assert st(n=24) == L.ERR_SHAPE
    assert st(s0=IN + 8) == L.ERR_SHAPE
    assert st(d0=IN + 16) == L.ERR_ALIAS
    assert st(d0=OUT, d1=OUT + 2048) == L.ERR_ALIAS
    assert st(n=0) == L.OK
    assert st(b=128) == L.ERR_VARIANT and st(u=2) == L.ERR_VARIANT
    assert st(g=0) == L.ERR_VARIANT and st(g=-3) == L.ERR_VARIANT and st(g=65537) == L.ERR_VARIANT
    assert st(n=0, g=65536) == L.OK


def test_static_scratch_covers_every_automatic_split():
    """The automatic choice never needs more workspace than the static
    scratch of skipln_forward_ws_static holds (256 KiB)."""
    lib = L.load()
    worst = 0
    for dt, v in ((L.F32, 4), (L.F16, 8)):
        for op in (L.OP_LAYER_NORM, L.OP_SIMPLIFIED, L.OP_BIAS_SOFTMAX):
            for mode, srows in ((L.SKIP_EXACT, 0), (L.SKIP_BROADCAST, 1)):
                for h in list(range(40904, 530000, v * 389)) + [65536, 81924, 163848, 262144, 524288]:
                    if h % v:
                        continue
                    worst = max(worst, lib.skipln_workspace_bytes(op, 10 ** 7, h, dt, mode, srows))
    assert 0 < worst < 154 * 1024


def test_static_entry_argument_checks():
    """skipln_forward_ws_static returns these before any HIP call."""
    st = lambda op=L.OP_LAYER_NORM, hidden=65536, rows=4, out=OUT, eps=1e-5, dtype=L.F32: \
        L.load().skipln_forward_ws_static(op, IN, SK, 0, 0, GA, BE, BI, out, RES, rows, hidden, eps, dtype, None)
    assert st(op=9) == L.ERR_OP
    assert st(dtype=5) == L.ERR_DTYPE
    assert st(eps=-1.0) == L.ERR_EPS
    assert st(hidden=0) == L.ERR_SHAPE
    assert st(out=None) == L.ERR_NULL
    assert st(out=IN + 4) == L.ERR_ALIAS
    assert st(rows=0) == L.OK


def test_rejected_arguments_raise_value_error():
    """The binding raises a SkiplnError for every status but SKIPLN_OK; a
    status that rejects the arguments is also a ValueError naming the
    status, one that reports the runtime or device is not."""
    import transformer_residual_add_amd as T

    L.check(L.OK, "ok")
    for st in (L.ERR_NULL, L.ERR_SHAPE, L.ERR_DTYPE, L.ERR_MODE, L.ERR_EPS, L.ERR_ALIAS, L.ERR_UNSUPPORTED,
               L.ERR_VARIANT, L.ERR_OP, L.ERR_WORKSPACE):
        with pytest.raises(ValueError) as e:
            L.check(st, "call")
        assert isinstance(e.value, L.SkiplnError) and e.value.status == st
        assert L.status_string(st) in str(e.value)
    for st in (L.ERR_LAUNCH, L.ERR_DEVICE):
        with pytest.raises(L.SkiplnError) as e:
            L.check(st, "call")
        assert not isinstance(e.value, ValueError)
    # host-only paths of the binding: an unknown element type, an unknown operation
    with pytest.raises(ValueError):
        T.workspace_bytes(L.OP_LAYER_NORM, 4, 64, 7)
    with pytest.raises(ValueError):
        T.workspace_bytes(9, 4, 64, L.F32)


def test_libraries_define_every_kernel_they_launch():
    """Neither library references a symbol of its own code that it does not
    define (a kernel whose launch stub the host pass dropped would show up
    here, and the library would not load)."""
    for path in (L.LIB_PATH, L.TUNE_LIB_PATH):
        out = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True, check=True).stdout
        assert not [ln for ln in out.splitlines() if "skipln" in ln], out
