"""Pins of the output-epilogue oracle (oracle/epilogue.py): the gated RMSNorm
y = o / sqrt(mean(o^2) + eps) * w * silu(g) against torch's own rms_norm and
silu in fp64, and closed forms that a dropped mean, a gate inside the norm or
a sigmoid in place of the SiLU would fail."""
import math

import numpy as np
import pytest
import torch

from oracle import epilogue as E


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("dv", [64, 128])
def test_matches_torch_rms_norm_and_silu(dv):
    o, g, w = _rand((5, 3, dv), 1), 2.0 * _rand((5, 3, dv), 2), _rand(dv, 3)
    for eps in (0.0, 1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(o), [dv], torch.from_numpy(w), eps) \
            * torch.nn.functional.silu(torch.from_numpy(g))
        assert np.abs(E.gated_rmsnorm(o, g, w, eps) - ref.numpy()).max() <= 1e-13


def test_constant_row_normalises_to_its_sign():
    dv = 64
    w = np.ones(dv)
    g = np.full(dv, 40.0)             # silu(40) = 40 (1 + e^-40)^-1, 40 to double precision
    for c in (3.0, -0.25):
        y = E.gated_rmsnorm(np.full(dv, c), g, w, 0.0)
        assert np.allclose(y, math.copysign(1.0, c) * 40.0 / (1.0 + math.exp(-40.0)), rtol=0, atol=1e-12)


def test_zero_gate_and_zero_row():
    o, w = _rand(128, 4), _rand(128, 5)
    assert np.array_equal(E.gated_rmsnorm(o, np.zeros(128), w, 1e-6), np.zeros(128))
    assert np.array_equal(E.gated_rmsnorm(np.zeros(128), _rand(128, 6), w, 1e-6), np.zeros(128))


def test_scale_invariance_and_unit_rms():
    o, g, w = _rand((4, 128), 7), _rand((4, 128), 8), _rand(128, 9)
    y = E.gated_rmsnorm(o, g, w, 0.0)
    assert np.allclose(E.gated_rmsnorm(37.5 * o, g, w, 0.0), y, rtol=1e-14, atol=0)
    z = y / (w * E.silu(g))                       # the normalised rows themselves
    assert np.allclose(np.mean(z * z, axis=-1), 1.0, rtol=1e-14)


def test_silu_values():
    assert E.silu(0.0) == 0.0
    assert abs(E.silu(math.log(3.0)) - 0.75 * math.log(3.0)) <= 1e-15
    assert abs(E.silu(-math.log(3.0)) + 0.25 * math.log(3.0)) <= 1e-15
