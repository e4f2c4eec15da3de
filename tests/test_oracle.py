"""The CPU oracle against its pins (closed forms, exhaustive binary16
conversion, exact-rational brute force, torch's float64 layer_norm,
invariants).  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()


def test_epsilon_default_is_binary32_of_1e_minus_12():
    """The manifest prints the default epsilon as a binary64; it is 1e-12
    rounded to binary32 (SkipLayerNormalization manifest, `attributes.epsilon`)."""
    with open(os.path.join(P.GOLDEN, "manifest_constants.json")) as fh:
        printed = json.load(fh)["epsilon_default"]["value"]
    assert float(np.float32(1e-12)) == printed


def test_oracle_rejects_bad_arguments():
    from oracle import oracle as O

    x = np.zeros((2, 4), np.float32)
    with pytest.raises(RuntimeError):
        O.skip_layer_norm(x, x, np.ones(4, np.float32), eps=-1.0)
    with pytest.raises(TypeError):
        O.skip_layer_norm(x, x.astype(np.float16), np.ones(4, np.float32))
    with pytest.raises(ValueError):
        O.skip_layer_norm(x, x[:1], np.ones(4, np.float32))
    r = O.skip_layer_norm(np.zeros((0, 4), np.float32), np.zeros((0, 4), np.float32), np.ones(4, np.float32))
    assert r["y"].shape == (0, 4)


def test_oracle_threads_agree():
    from oracle import oracle as O

    rng = np.random.default_rng(0)
    x = rng.standard_normal((37, 130)).astype(np.float32)
    s = rng.standard_normal((37, 130)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 130).astype(np.float32)
    a = O.skip_layer_norm(x, s, g, threads=1)
    b = O.skip_layer_norm(x, s, g, threads=5)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["residual"], b["residual"])
