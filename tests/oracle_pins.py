"""Pins for the CPU oracle: checks against what the operator's definition and
mathematics fix, independent of the oracle's own code.

Each ``check_*`` function raises AssertionError on a mismatch.  They are run
against the real oracle (tests/test_oracle.py) and against copies of the
oracle with a planted mistake (tests/test_oracle_mutants.py), which must each
fail at least one check.

Definition pinned: com.microsoft SkipLayerNormalization WebGPU manifest --
`description`, `inputs[skip]`, `inputs[bias]`, `inputs[gamma]`,
`inputs[beta]`, `outputs[input_skip_bias_sum]`, `attributes.epsilon` and
`attributeDescriptions.epsilon`; float16 per `typeConstraints.T` and the
IEEE 754 binary16 format.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NP = {"f32": np.float32, "f16": np.float16}


# ---------------------------------------------------------------- helpers --

def _arr(v, dt):
    return None if v is None else np.asarray(v, dtype=np.float64).astype(dt)


def _close(got, want, atol, rtol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{what}: NaN pattern differs"
    g, w = got[~nan_w], want[~nan_w]
    err = np.abs(g - w)
    bad = err > atol + rtol * np.abs(w)
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} of {bad.size} outside {atol}+{rtol}*|want|; "
        f"max err {err.max():.3e}"
    )


def _eval_closed_form(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"sqrt": math.sqrt, "nan": float("nan")}))


def _f32_sum(x, skip_rows_view, bias):
    """Pre-normalization sum with numpy's IEEE binary32 adds, in the order
    (input + skip) + bias -- an independent library computation."""
    s = x.astype(np.float32) + skip_rows_view.astype(np.float32)
    if bias is not None:
        s = s + bias.astype(np.float32)
    return s


# ------------------------------------------------------------ conversions --

def check_f16_decode_exhaustive():
    """All 65536 binary16 patterns decode like numpy's float16 -> float32."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.f16_to_f32(bits)
    want = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN decode differs"
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32)), \
        "binary16 decode differs from numpy"


def _f16_encode_candidates(rng):
    fin = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)  # finite, positive
    vals = fin.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # exact in binary32 (12 significant bits)
    base = np.concatenate([vals, mids, [65504.0, 65519.0, 65520.0, 65535.0, 65536.0, 1e6,
                                        2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26,
                                        2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1e-30, 0.0]])
    f = base.astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(0))
    rnd = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32).view(np.float32)
    allv = np.concatenate([f, up, dn, rnd, np.array([np.inf, np.nan], np.float32)])
    return np.concatenate([allv, -allv])


def check_f16_encode():
    """binary32 -> binary16 encodes like numpy (round to nearest, ties to even)
    on every binary16 value, every midpoint between neighbours, one binary32
    step either side of each, the overflow/underflow edges and 2^20 random
    binary32 patterns."""
    rng = np.random.default_rng(12345)
    f = _f16_encode_candidates(rng)
    with np.errstate(over="ignore", invalid="ignore"):
        want = f.astype(np.float16)
    got = O.f32_to_f16(f)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got.view(np.float16)), nan), "NaN encode differs"
    diff = got[~nan] != want[~nan].view(np.uint16)
    assert not diff.any(), f"{int(diff.sum())} binary16 encodings differ, e.g. {f[~nan][diff][:4]}"


# ------------------------------------------------------------- hand rows --

def check_hand_rows():
    with open(os.path.join(GOLDEN, "hand_rows.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        dt = NP[c["dtype"]]
        x = _arr(c["input"], dt)
        skip = _arr(c["skip"], dt)
        bcast = c["skip_rows"] > 0
        r = O.skip_layer_norm(x, skip, _arr(c["gamma"], dt), _arr(c["beta"], dt), _arr(c["bias"], dt),
                              c["eps"], broadcast=bcast, stats=True)
        name = c["name"]
        if "y" in c:
            want = [[_eval_closed_form(e) for e in row] for row in c["y"]]
            _close(r["y"], want, 1e-14, 1e-14, f"{name}: y")
        if "mean" in c:
            _close(r["mean"], [float(Fraction(m)) for m in c["mean"]], 1e-15, 1e-15, f"{name}: mean")
            _close(r["var"], [float(Fraction(v)) for v in c["var"]], 1e-15, 1e-15, f"{name}: var")
        if "residual" in c:
            assert np.array_equal(r["residual"].astype(np.float64), np.asarray(c["residual"], np.float64)), \
                f"{name}: residual"
        if "residual_bits" in c:
            want_bits = np.array([[int(b, 16) for b in row] for row in c["residual_bits"]], np.uint16)
            assert np.array_equal(r["residual"].view(np.uint16), want_bits), \
                f"{name}: residual bits {r['residual'].view(np.uint16)} != {want_bits}"


# ----------------------------------------------------------- brute force --

getcontext().prec = 50


def _exact_row(s_row, gamma, beta, eps_f):
    """Exact rational mean and variance; the normalized row to 50 digits."""
    h = len(s_row)
    s = [Fraction(float(v)) for v in s_row]
    m = sum(s, Fraction(0)) / h
    var = sum(((v - m) ** 2 for v in s), Fraction(0)) / h
    den2 = var + Fraction(eps_f)
    out = []
    for v, g, b in zip(s, gamma, beta):
        if den2 == 0:
            out.append(float("nan"))
            continue
        d = Decimal((v - m).numerator) / Decimal((v - m).denominator)
        q = Decimal(den2.numerator) / Decimal(den2.denominator)
        z = d / q.sqrt()
        out.append(float(z * Decimal(float(g)) + Decimal(float(b))))
    return m, var, out


def check_bruteforce_2x4(n_cases: int = 300):
    """2 x 4 problems on dyadic inputs whose sums are exact in float16 and
    float32: exact rational statistics and a 50-digit normalized output
    against the oracle, over every flag combination, both skip forms and
    both I/O types."""
    rng = np.random.default_rng(2024)
    for k in range(n_cases):
        dt = np.float32 if k % 2 == 0 else np.float16
        bcast = (k // 2) % 2 == 1
        has_beta, has_bias = (k // 4) % 2 == 1, (k // 8) % 2 == 1
        eps = [0.0, 2.0 ** -10, 0.25, 1e-5][(k // 16) % 4]
        rows, h = 2, 4
        x = (rng.integers(-64, 65, (rows, h)) / 8.0).astype(dt)
        sk_rows = 1 if bcast else rows
        skip = (rng.integers(-64, 65, (sk_rows, h)) / 8.0).astype(dt)
        gamma = rng.choice([0.5, 0.75, 1.0, 1.25, 1.5, -1.0], h).astype(dt)
        beta = (rng.integers(-16, 17, h) / 16.0).astype(dt) if has_beta else None
        bias = (rng.integers(-16, 17, h) / 16.0).astype(dt) if has_bias else None
        r = O.skip_layer_norm(x, skip, gamma, beta, bias, eps, broadcast=bcast, stats=True)
        eps_f = float(np.float32(eps))
        for i in range(rows):
            j = i % sk_rows
            s = [float(x[i, c]) + float(skip[j, c]) + (float(bias[c]) if has_bias else 0.0) for c in range(h)]
            assert np.array_equal(r["residual"][i].astype(np.float64), np.array(s)), f"case {k}: residual row {i}"
            m, var, y = _exact_row(s, gamma, beta if has_beta else [0.0] * h, eps_f)
            _close(r["mean"][i], float(m), 1e-15, 1e-15, f"case {k}: mean row {i}")
            _close(r["var"][i], float(var), 1e-15, 1e-14, f"case {k}: var row {i}")
            _close(r["y"][i], y, 1e-13, 1e-13, f"case {k}: y row {i}")


# ---------------------------------------------------- library special case --

def check_torch_layer_norm():
    """The normalization step equals torch's float64 layer_norm applied to the
    binary32 sum formed by numpy (an independent textbook implementation)."""
    import torch

    rng = np.random.default_rng(77)
    for dt, h, rows, bcast, has_bias, has_beta, eps in [
        (np.float32, 768, 64, False, True, True, 1e-12),
        (np.float32, 100, 48, True, False, True, 1e-5),
        (np.float16, 1024, 32, False, True, True, 1e-5),
        (np.float16, 37, 24, True, True, False, 0.1),
    ]:
        x = (100 * (dt == np.float16) + rng.standard_normal((rows, h))).astype(dt)
        sk_rows = 8 if bcast else rows
        skip = rng.standard_normal((sk_rows, h)).astype(dt)
        gamma = rng.uniform(0.5, 1.5, h).astype(dt)
        beta = (0.1 * rng.standard_normal(h)).astype(dt) if has_beta else None
        bias = (0.1 * rng.standard_normal(h)).astype(dt) if has_bias else None
        r = O.skip_layer_norm(x, skip, gamma, beta, bias, eps, broadcast=bcast)
        s = _f32_sum(x, skip[np.arange(rows) % sk_rows], bias)
        want = torch.nn.functional.layer_norm(
            torch.from_numpy(s.astype(np.float64)), (h,),
            weight=torch.from_numpy(gamma.astype(np.float64)),
            bias=None if beta is None else torch.from_numpy(beta.astype(np.float64)),
            eps=float(np.float32(eps)),
        ).numpy()
        _close(r["y"], want, 1e-12, 1e-12, f"torch layer_norm {dt.__name__} H={h}")


# -------------------------------------------------------------- residual --

def check_residual():
    """Residual = numpy binary32 adds (input + skip) + bias, rounded once to T;
    without bias it is the correctly rounded exact sum."""
    rng = np.random.default_rng(5)
    for dt in (np.float32, np.float16):
        for has_bias in (False, True):
            rows, h = 40, 96
            x = rng.standard_normal((rows, h)).astype(dt)
            skip = (0.5 * rng.standard_normal((rows, h))).astype(dt)
            bias = (0.1 * rng.standard_normal(h)).astype(dt) if has_bias else None
            gamma = np.ones(h, dt)
            r = O.skip_layer_norm(x, skip, gamma, None, bias, 1e-5)
            want = _f32_sum(x, skip, bias).astype(dt)
            assert np.array_equal(r["residual"].view(np.uint8), want.view(np.uint8)), \
                f"residual {dt.__name__} bias={has_bias}"
            if not has_bias:
                # correctly rounded exact sum of two T values, element by element
                for i in range(0, rows, 7):
                    for c in range(0, h, 5):
                        ex = Fraction(float(x[i, c])) + Fraction(float(skip[i, c]))
                        cr = np.float64(float(ex)).astype(dt) if dt == np.float16 else np.float32(float(ex))
                        assert float(r["residual"][i, c]) == float(cr), f"exact sum {dt.__name__} ({i},{c})"


# ------------------------------------------------------------ invariants --

def _dyadic(rng, shape, dt, scale=8):
    return (rng.integers(-8 * scale, 8 * scale + 1, shape) / scale).astype(dt)


def check_invariants():
    rng = np.random.default_rng(99)
    rows, h = 12, 64
    for dt in (np.float32, np.float16):
        x = _dyadic(rng, (rows, h), dt)
        skip = _dyadic(rng, (rows, h), dt)
        bias = _dyadic(rng, (h,), dt, 16)
        gamma = rng.uniform(0.5, 1.5, h).astype(dt)
        beta = (0.1 * rng.standard_normal(h)).astype(dt)
        eps = 1e-5
        base = O.skip_layer_norm(x, skip, gamma, beta, bias, eps, stats=True)

        # (a) adding a constant to a whole input row leaves the output unchanged
        shifted = O.skip_layer_norm((x.astype(np.float64) + 4.0).astype(dt), skip, gamma, beta, bias, eps)
        _close(shifted["y"], base["y"], 1e-12, 1e-12, "shift invariance")

        # (b) gamma = 1, beta = 0: each row has mean 0 and variance var/(var+eps)
        big_eps = 0.25
        unit = O.skip_layer_norm(x, skip, np.ones(h, dt), None, bias, big_eps, stats=True)
        _close(unit["y"].mean(axis=1), np.zeros(rows), 1e-13, 0, "normalized row mean")
        _close(unit["y"].var(axis=1), unit["var"] / (unit["var"] + big_eps), 1e-13, 1e-13,
               "normalized row variance")

        # (c) positive power-of-two scaling of the row with eps = 0 changes nothing
        s0 = O.skip_layer_norm(x, skip, gamma, beta, bias, 0.0)
        s1 = O.skip_layer_norm((x.astype(np.float64) * 2).astype(dt), (skip.astype(np.float64) * 2).astype(dt),
                               gamma, beta, (bias.astype(np.float64) * 2).astype(dt), 0.0)
        _close(s1["y"], s0["y"], 1e-13, 1e-13, "scale invariance")

        # (d) permuting the columns of every operand permutes the output
        p = rng.permutation(h)
        perm = O.skip_layer_norm(x[:, p], skip[:, p], gamma[p], beta[p], bias[p], eps)
        _close(perm["y"], base["y"][:, p], 1e-13, 1e-13, "column permutation")

        # (e) rows are independent: perturbing row 3 changes no other row
        x2 = x.copy()
        x2[3] = (x2[3].astype(np.float64) * -3 + 1).astype(dt)
        pert = O.skip_layer_norm(x2, skip, gamma, beta, bias, eps)
        others = np.arange(rows) != 3
        assert np.array_equal(pert["y"][others], base["y"][others]), "row independence"
        assert not np.allclose(pert["y"][3], base["y"][3]), "perturbed row unchanged"

        # (f) broadcast skip == exact skip tiled across the batch
        S = 4
        sk = skip[:S]
        bc = O.skip_layer_norm(x, sk, gamma, beta, bias, eps, broadcast=True)
        ex = O.skip_layer_norm(x, np.tile(sk, (rows // S, 1)), gamma, beta, bias, eps)
        assert np.array_equal(bc["y"], ex["y"]) and np.array_equal(bc["residual"], ex["residual"]), \
            "broadcast vs tiled"

        # (g) a row block with row_offset equals the same rows of the whole
        part = O.skip_layer_norm(x[5:11], sk, gamma, beta, bias, eps, broadcast=True, row_offset=5)
        assert np.array_equal(part["y"], bc["y"][5:11]), "row_offset block"

        # (h) bias folds into the skip: (x + skip) + bias == x + (skip + bias) on exact data
        fold = O.skip_layer_norm(x, (skip.astype(np.float64) + bias).astype(dt), gamma, beta, None, eps)
        _close(fold["y"], base["y"], 1e-13, 1e-13, "bias folding")

        # (i) beta shifts, gamma scales the normalized value column by column
        nob = O.skip_layer_norm(x, skip, np.ones(h, dt), None, bias, eps)
        _close(base["y"], nob["y"] * gamma.astype(np.float64) + beta.astype(np.float64), 1e-13, 1e-13,
               "affine step")


def check_cancellation_rows():
    """Rows with mean ~100 and variance ~2 (float16): the oracle's binary64
    variance matches the exact rational variance of the same binary32 sums."""
    rng = np.random.default_rng(31)
    rows, h = 6, 8192
    x = (100 + rng.standard_normal((rows, h))).astype(np.float16)
    skip = rng.standard_normal((rows, h)).astype(np.float16)
    bias = (0.1 * rng.standard_normal(h)).astype(np.float16)
    gamma = rng.uniform(0.5, 1.5, h).astype(np.float16)
    r = O.skip_layer_norm(x, skip, gamma, None, bias, 1e-5, stats=True)
    s = _f32_sum(x, skip, bias)
    for i in range(rows):
        fr = [Fraction(float(v)) for v in s[i]]
        m = sum(fr, Fraction(0)) / h
        var = sum(((v - m) ** 2 for v in fr), Fraction(0)) / h
        assert abs(r["mean"][i] - float(m)) <= 1e-12 * abs(float(m)), "cancellation mean"
        assert abs(r["var"][i] - float(var)) <= 1e-12 * float(var), "cancellation variance"


# ---------------------------------------------------------------- simplified --

def check_simplified():
    """Root-mean-square form: no mean subtraction, the mean square under the
    square root; hand rows and the invariant that each gamma=1 row has mean
    square ms/(ms+eps)."""
    x = np.array([[3.0, 4.0], [1.0, -1.0]], np.float32)
    z = np.zeros_like(x)
    r = O.skip_layer_norm(x, z, np.ones(2, np.float32), None, None, 0.0, simplified=True, stats=True)
    # row 0: mean square (9+16)/2 = 12.5 -> y = [3, 4]/sqrt(12.5); row 1: ms 1 -> y = [1, -1]
    _close(r["y"], [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], [1.0, -1.0]], 1e-15, 1e-15, "rms hand rows")
    _close(r["var"], [12.5, 1.0], 0, 1e-15, "rms mean square")
    rng = np.random.default_rng(8)
    x = rng.standard_normal((8, 50)).astype(np.float32)
    r = O.skip_layer_norm(x, np.zeros_like(x), np.ones(50, np.float32), None, None, 0.5,
                          simplified=True, stats=True)
    _close((r["y"] ** 2).mean(axis=1), r["var"] / (r["var"] + 0.5), 1e-13, 1e-13, "rms invariant")


# ---------------------------------------------------------------- BiasAdd --

def check_bias_add():
    """BiasAdd: Y = (X + bias) + skip with binary32 adds in that order, rounded
    once to T (com.microsoft BiasAdd manifest, `description`)."""
    rng = np.random.default_rng(3)
    for dt in (np.float32, np.float16):
        x = rng.standard_normal((2, 5, 24)).astype(dt)
        skip = rng.standard_normal((2, 5, 24)).astype(dt)
        bias = rng.standard_normal(24).astype(dt)
        y, ye = O.bias_add(x, bias, skip)
        want = ((x.astype(np.float32) + bias.astype(np.float32)) + skip.astype(np.float32)).astype(dt)
        assert np.array_equal(y.view(np.uint8), want.view(np.uint8)), f"bias_add {dt.__name__}"
        exact = x.astype(np.float64) + bias.astype(np.float64) + skip.astype(np.float64)
        _close(ye, exact, 1e-15, 1e-15, "bias_add exact")


def check_bias_add_hand_rows():
    """Hand-derived BiasAdd rows (tests/golden/bias_add_rows.json), among them
    rows whose binary32 result depends on the grouping: X + bias first, then
    the skip (com.microsoft BiasAdd manifest, `description`)."""
    with open(os.path.join(GOLDEN, "bias_add_rows.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        dt = NP[c["dtype"]]
        y, _ = O.bias_add(_arr(c["x"], dt), _arr(c["bias"], dt), _arr(c["skip"], dt))
        if "y" in c:
            assert np.array_equal(y.astype(np.float64), np.asarray(c["y"], np.float64)), \
                f"{c['name']}: Y {y.tolist()} != {c['y']}"
        if "y_bits" in c:
            want = np.array([[int(b, 16) for b in row] for row in c["y_bits"]], np.uint16)
            assert np.array_equal(y.view(np.uint16), want), f"{c['name']}: Y bits {y.view(np.uint16)} != {want}"


# ------------------------------------------------------------ BiasSoftmax --

def check_bias_softmax_closed_forms():
    """BiasSoftmax (com.microsoft BiasSoftmax manifest, `description`,
    `attributeDescriptions.is_inner_broadcast`, `derive.biasContract`):
    softmax([0, a]) is the logistic pair (1/(1+e^a), e^a/(1+e^a)); a constant
    row is uniform; a row offset by 1000 is unchanged (the maximum is taken
    out before exponentiating); bias rows are reused in consecutive groups
    (inner) or cyclically (outer)."""
    f32 = np.float32
    a = f32(0.75)
    y = O.bias_softmax(np.array([[0.0, a]], f32), np.zeros((1, 2), f32), True)
    e = math.exp(float(a))
    _close(y, [[1 / (1 + e), e / (1 + e)]], 1e-16, 1e-15, "logistic pair")
    y = O.bias_softmax(np.full((3, 5), 2.5, f32), np.zeros((1, 5), f32), False)
    _close(y, np.full((3, 5), 0.2), 1e-16, 1e-15, "constant rows")
    ln3 = f32(math.log(3.0))
    e3 = math.exp(float(ln3))
    y = O.bias_softmax(np.array([[1000.0, 1000.0 + float(ln3)]], f32), np.zeros((1, 2), f32), True)
    z1 = float(f32(1000.0 + float(ln3))) - 1000.0  # the binary32 input is what the row holds
    _close(y, [[1 / (1 + math.exp(z1)), math.exp(z1) / (1 + math.exp(z1))]], 1e-15, 1e-14, "offset row")
    # The maximum is not the first value and e^800 overflows binary64: only
    # subtracting the true maximum gives the closed form [~0, 1].
    y = O.bias_softmax(np.array([[0.0, 800.0]], f32), np.zeros((1, 2), f32), True)
    _close(y, [[0.0, 1.0]], 1e-300, 1e-15, "maximum last, large spread")
    # Two bias rows [0, ln3] and [ln3, 0] over four zero data rows.
    bias = np.array([[0.0, ln3], [ln3, 0.0]], f32)
    lo, hi = 1 / (1 + e3), e3 / (1 + e3)
    y_in = O.bias_softmax(np.zeros((4, 2), f32), bias, True)
    _close(y_in, [[lo, hi], [lo, hi], [hi, lo], [hi, lo]], 1e-16, 1e-15, "inner broadcast groups")
    y_out = O.bias_softmax(np.zeros((4, 2), f32), bias, False)
    _close(y_out, [[lo, hi], [hi, lo], [lo, hi], [hi, lo]], 1e-16, 1e-15, "outer broadcast cycles")
    # a NaN or a fully masked (-inf) row gives NaN, in that row only
    d = np.zeros((3, 4), f32)
    d[1, 2] = np.nan
    d[2, :] = -np.inf
    y = O.bias_softmax(d, np.zeros((1, 4), f32), True)
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all() and not np.isnan(y[0]).any(), "NaN rows"


def check_bias_softmax_libraries():
    """torch's and scipy's float64 softmax of the binary32 sum formed by numpy."""
    import scipy.special
    import torch

    rng = np.random.default_rng(17)
    for dt, rows, cols, brows, inner in [(np.float32, 24, 512, 4, True), (np.float32, 18, 77, 6, False),
                                         (np.float16, 32, 256, 8, True), (np.float16, 12, 1000, 3, False)]:
        data = (3 * rng.standard_normal((rows, cols))).astype(dt)
        bias = (rng.standard_normal((brows, cols)) - 2 * (rng.random((brows, cols)) < 0.3)).astype(dt)
        rep = rows // brows
        idx = np.arange(rows) // rep if inner else np.arange(rows) % brows
        z = (data.astype(np.float32) + bias[idx].astype(np.float32)).astype(np.float64)
        y = O.bias_softmax(data, bias, inner)
        _close(y, torch.softmax(torch.from_numpy(z), dim=1).numpy(), 1e-15, 1e-12, "torch softmax")
        _close(y, scipy.special.softmax(z, axis=1), 1e-15, 1e-12, "scipy softmax")


def check_bias_softmax_invariants():
    rng = np.random.default_rng(23)
    data = (rng.integers(-40, 41, (12, 33)) / 8).astype(np.float32)
    bias = (rng.integers(-40, 41, (4, 33)) / 8).astype(np.float32)
    for inner in (True, False):
        y = O.bias_softmax(data, bias, inner)
        _close(y.sum(axis=1), np.ones(12), 1e-14, 0, "rows sum to 1")
        # ratios follow exp of differences (dyadic data: the sums are exact)
        rep = 12 // 4
        idx = np.arange(12) // rep if inner else np.arange(12) % 4
        z = data.astype(np.float64) + bias[idx].astype(np.float64)
        _close(y[:, 1:] / y[:, :1], np.exp(z[:, 1:] - z[:, :1]), 0, 1e-13, "ratios")
        # adding a constant to a data row changes nothing
        y2 = O.bias_softmax((data.astype(np.float64) + 4.0).astype(np.float32), bias, inner)
        _close(y2, y, 1e-15, 1e-13, "shift invariance")
    # one bias row for all: inner and outer agree
    b1 = bias[:1]
    assert np.array_equal(O.bias_softmax(data, b1, True), O.bias_softmax(data, b1, False)), "single bias row"


ALL_CHECKS = [
    check_f16_decode_exhaustive,
    check_f16_encode,
    check_hand_rows,
    check_bruteforce_2x4,
    check_torch_layer_norm,
    check_residual,
    check_invariants,
    check_cancellation_rows,
    check_simplified,
    check_bias_add_hand_rows,
    check_bias_add,
    check_bias_softmax_closed_forms,
    check_bias_softmax_libraries,
    check_bias_softmax_invariants,
]
