"""The oracle's float16 residual against the exact sum, over every row of the
two float16 workloads (16384 x 1024 and 65536 x 8192, both with a bias).
CPU only.

The residual (SkipLayerNormalization manifest, `outputs[input_skip_bias_sum]`)
is the binary32 sum (input + skip) + bias rounded once to float16.  The exact
sum of three float16 values is exact in binary64 (their significands span at
most 2^-24 .. 2^16, 41 bits), and numpy rounds binary64 to float16 correctly,
so round16(exact) is computed here without the oracle's arithmetic.

Without a bias the two agree everywhere: binary32 has 24 >= 2*11 + 2
significand bits, so rounding first to binary32 and then to float16 gives the
correctly rounded float16 value (double rounding is innocuous under that
condition).  With a bias the sum takes two binary32 roundings, and the float16
result may differ from round16(exact) where the exact sum lies within those
roundings of a float16 rounding boundary.  The test reports how many elements
differ and requires each difference to be of that kind: the two float16 values
are neighbours and the exact sum lies within one binary32 unit in the last
place of their midpoint.
"""
import numpy as np
import pytest

from oracle import oracle as O
from transformer_residual_add_amd import workloads as W

BLOCK = 4096


def _explained(exact, got16, want16):
    """Whether every difference is a float16 rounding-boundary case."""
    gb = got16.view(np.uint16).astype(np.int32)
    wb = want16.view(np.uint16).astype(np.int32)
    same_sign = (gb & 0x8000) == (wb & 0x8000)
    neighbours = same_sign & (np.abs(gb - wb) == 1)
    mid = 0.5 * (got16.astype(np.float64) + want16.astype(np.float64))
    # one binary32 unit in the last place at the larger of |exact| and |mid|
    mag = np.maximum(np.abs(exact), np.abs(mid))
    ulp32 = np.spacing(mag.astype(np.float32)).astype(np.float64)
    near = np.abs(exact - mid) <= ulp32
    return neighbours & near


@pytest.mark.parametrize("name", ["rows16384_h1024_f16", "rows65536_h8192_f16_mean100"])
def test_float16_residual_is_the_rounded_exact_sum(name):
    w = W.WORKLOADS[name]
    assert w.dtype == "f16" and w.residual and w.bias_dist is not None
    no_bias = 0
    differ = 0
    checked = 0
    for r0 in range(0, w.rows, BLOCK):
        r1 = min(w.rows, r0 + BLOCK)
        part = W.make_rows(w, r0, r1)
        x, sk, b = part["input"], part["skip"], part["bias"]
        exact = x.astype(np.float64) + sk.astype(np.float64) + b.astype(np.float64)[None, :]
        want = exact.astype(np.float16)
        got = O.skip_layer_norm(x, sk, part["gamma"], part["beta"], b, w.eps, residual=True, threads=8)["residual"]
        d = got.view(np.uint16) != want.view(np.uint16)
        n = int(d.sum())
        if n:
            ok = _explained(exact[d], got[d], want[d])
            assert ok.all(), (f"{name} rows {r0}:{r1}: {int((~ok).sum())} residuals differ from the rounded exact "
                              f"sum by more than a rounding-boundary case")
        differ += n
        checked += d.size
        # Without the bias, the rounded binary32 sum is the rounded exact sum.
        exact2 = x.astype(np.float64) + sk.astype(np.float64)
        got2 = O.skip_layer_norm(x[:64], sk[:64], part["gamma"], None, None, w.eps, residual=True)["residual"]
        no_bias += int((got2.view(np.uint16) != exact2[:64].astype(np.float16).view(np.uint16)).sum())
    print(f"{name}: {differ} of {checked} float16 residuals differ from round16(exact sum) "
          f"({differ / checked:.2e}), each a rounding-boundary case; without the bias 0 expected, {no_bias} found")
    assert no_bias == 0
    # Rare: a difference needs the exact sum within ~2^-24 relative of a
    # float16 midpoint, one element in ~2^12 or fewer.
    assert differ <= checked // 1024
