"""The seeded synthetic inputs: the five workload configurations (shapes,
element types, skip forms, optional tensors, epsilon, value laws), and the
same seed giving the same bytes whatever the thread count or the slice of
rows regenerated.  No operator arithmetic here: the generators only draw
values and round them once to the element type."""
import hashlib

import numpy as np
import pytest

from transformer_residual_add_amd import workloads as W

# name: (logical shape, skip shape, dtype, bias, residual, epsilon, input law (mu, sigma), skip law)
CONFIGS = {
    "tiny_2x8x64_f32": ((2, 8, 64), (2, 8, 64), "f32", False, False, 1e-12, (0, 1), (0, 1)),
    "bert_base_8x128x768_f32": ((8, 128, 768), (8, 128, 768), "f32", True, True, 1e-12, (0, 1), (0, 0.5)),
    "rows16384_h1024_f16": ((16384, 1024), (16384, 1024), "f16", True, True, 1e-5, (0, 1), (0, 1)),
    "bcast_64x512x4096_f32": ((64, 512, 4096), (512, 4096), "f32", False, False, 1e-12, (0, 1), (0, 1)),
    "rows65536_h8192_f16_mean100": ((65536, 8192), (65536, 8192), "f16", True, True, 1e-5, (100, 1), (0, 1)),
}


def digest(arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(b"-" if a is None else np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_the_five_configurations():
    assert W.ORDER == list(CONFIGS)
    for name, (shape, skip_shape, dt, bias, residual, eps, _, _) in CONFIGS.items():
        w = W.WORKLOADS[name]
        assert (w.shape, w.skip_shape, w.dtype, w.residual, w.eps) == (shape, skip_shape, dt, residual, eps), name
        assert (w.bias_dist is not None) == bias, name
        assert w.gamma_dist is not None and w.beta_dist is not None, name   # gamma U(0.5,1.5), beta N(0,0.1)
        assert w.broadcast == (skip_shape != shape), name
        assert w.rows == int(np.prod(shape[:-1])) and w.hidden == shape[-1]
        assert w.skip_rows == int(np.prod(skip_shape[:-1]))


@pytest.mark.parametrize("name", ["tiny_2x8x64_f32", "bert_base_8x128x768_f32"])
def test_same_seed_same_bytes(name):
    w = W.WORKLOADS[name]
    a = W.make_inputs(w, threads=1)
    b = W.make_inputs(w, threads=4)
    keys = ("input", "skip", "bias", "gamma", "beta")
    assert digest(a[k] for k in keys) == digest(b[k] for k in keys)
    for k in keys:
        if a[k] is not None:
            assert a[k].dtype == w.np_dtype and a[k].flags.c_contiguous


def test_row_slices_regenerate_the_same_rows():
    """make_rows(r0, r1) is bit-identical to the same rows of make_inputs,
    across the 256-row generation blocks, for exact and broadcast skips."""
    for w in (W.WORKLOADS["bert_base_8x128x768_f32"],
              W.WORKLOADS["bcast_64x512x4096_f32"].with_(shape=(3, 512, 256), skip_shape=(512, 256))):
        full = W.make_inputs(w)
        for r0, r1 in ((0, 1), (255, 257), (300, 812), (w.rows - 3, w.rows)):
            part = W.make_rows(w, r0, r1)
            assert np.array_equal(part["input"].view(np.uint8), full["input"][r0:r1].view(np.uint8))
            if w.broadcast:
                assert np.array_equal(part["skip"], full["skip"])
            else:
                assert np.array_equal(part["skip"].view(np.uint8), full["skip"][r0:r1].view(np.uint8))


@pytest.mark.parametrize("name", ["bert_base_8x128x768_f32", "rows16384_h1024_f16"])
def test_value_laws(name):
    """Sample moments of the drawn tensors against the stated laws, and every
    value representable in the element type (drawn in binary64, rounded once)."""
    w = W.WORKLOADS[name]
    _, _, _, _, _, _, (mu_x, sd_x), (mu_s, sd_s) = CONFIGS[name]
    inp = W.make_inputs(w)
    for key, mu, sd in (("input", mu_x, sd_x), ("skip", mu_s, sd_s)):
        v = inp[key].astype(np.float64)
        n = v.size
        assert abs(v.mean() - mu) < 5 * sd / np.sqrt(n) + 1e-3 * sd, key
        assert abs(v.std() / sd - 1) < 0.01, key
    g = inp["gamma"].astype(np.float64)
    assert g.min() >= 0.5 and g.max() <= 1.5 and abs(g.mean() - 1) < 0.05
    assert abs(inp["beta"].astype(np.float64).std() / 0.1 - 1) < 0.15
    for key in ("input", "skip", "bias", "gamma", "beta"):
        a = inp[key]
        if a is not None:
            assert np.array_equal(a.astype(np.float64).astype(a.dtype), a), key


def test_large_mean_rows_hold_the_offset():
    """The mean-100 workload: rows drawn around 100 (variance cancellation),
    checked on regenerated row blocks without building the 1 GiB tensor."""
    w = W.WORKLOADS["rows65536_h8192_f16_mean100"]
    part = W.make_rows(w, 4096, 4096 + 64)
    x = part["input"].astype(np.float64)
    assert abs(x.mean() - 100) < 0.01 and abs(x.std() - 1) < 0.02
    assert part["input"].dtype == np.float16
