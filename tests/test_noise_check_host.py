"""The noise-floor gate of the GPU tests (CPU only): it accepts an independent
draw of the rounding model's error and rejects a small systematic extra."""
import importlib.util
import os

import numpy as np
import pytest

_spec = importlib.util.spec_from_file_location(
    "_noise_floor", os.path.join(os.path.dirname(__file__), "test_gpu_noise_floor.py"))
nf = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(nf)


def _draws(seed, n=200000):
    rng = np.random.default_rng(seed)
    out = rng.normal(0.0, 0.05, n)                       # outputs of a long-context batch
    # two independent roundings of the same values to bf16 (one ulp apart at most)
    jitter = rng.uniform(-1, 1, (2, n)) * 2.0 ** -10 * np.abs(out)
    a = nf.bf16_round(out + jitter[0]) - out
    b = nf.bf16_round(out + jitter[1]) - out
    return out, a, b


def test_bf16_round_ties_to_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.1, 3.0e-40])
    got = nf.bf16_round(x)
    assert got[0] == 1.0 and got[1] == 1.0 + 2.0 ** -6   # ties to the even neighbour
    assert abs(got[2] + 0.1) < 2.0 ** -9 * 0.1
    assert got[3] >= 0.0


def test_independent_rounding_draws_pass():
    _, a, b = _draws(1)
    nf._check(a, b, "independent draws")


def test_systematic_extra_error_fails():
    out, a, b = _draws(2)
    extra = a + 2.0 ** -9 * out                          # one extra relative rounding-sized term
    with pytest.raises(AssertionError):
        nf._check(extra, b, "systematic extra")
