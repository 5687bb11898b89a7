"""Pins of the oracle's gate/up activation (oracle/act.py) against closed forms
of the logistic function and the half-split structure of the fused w13
output, each chosen so that a plausible slip fails: sigmoid(-z) in place of
sigmoid(z), the gate and up halves swapped, a missing factor, overflow at
large |z|."""

import math

import numpy as np
import pytest

import oracle


def test_silu_closed_forms():
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly; sigmoid(0) = 1/2
    ln3 = math.log(3.0)
    got = oracle.silu(np.array([0.0, ln3, -ln3, math.log(7.0)]))
    want = np.array([0.0, 0.75 * ln3, -0.25 * ln3, 0.875 * math.log(7.0)])
    assert np.allclose(got, want, rtol=1e-15, atol=0)


def test_silu_symmetry_and_limits():
    z = np.linspace(-30, 30, 601)
    # silu(z) - silu(-z) = z * (sigmoid(z) + sigmoid(-z)) = z
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-13)
    # large positive: silu(z) = z up to e^-z; large negative: a signed zero or tiny
    big = oracle.silu(np.array([800.0, -800.0, 40.0]))
    assert big[0] == 800.0 and big[1] == 0.0 and abs(big[2] - 40.0) < 1e-15
    # the global minimum of silu is near z = -1.2785 with value -0.27846
    zz = np.linspace(-3, 0, 300001)
    i = int(np.argmin(oracle.silu(zz)))
    assert abs(zz[i] + 1.27846) < 1e-4 and abs(oracle.silu(zz[i]) + 0.278465) < 1e-5


def test_silu_mul_half_split():
    # gate = ln 3, up = 4  ->  3 ln 3; swapping halves would give silu(4) ln 3
    y = np.array([[math.log(3.0), 0.0, 4.0, 5.0]])
    h = oracle.silu_mul(y)
    assert h.shape == (1, 2)
    assert abs(h[0, 0] - 3.0 * math.log(3.0)) < 1e-14
    assert h[0, 1] == 0.0
    # up = 1 reduces to silu of the gate half
    g = np.random.default_rng(0).standard_normal((5, 8))
    assert np.array_equal(oracle.silu_mul(np.concatenate([g, np.ones_like(g)], axis=1)),
                          oracle.silu(g))
    with pytest.raises(ValueError):
        oracle.silu_mul(np.zeros((2, 3)))
