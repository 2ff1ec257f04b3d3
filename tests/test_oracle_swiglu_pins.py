"""Pins for the oracle's gated-MLP epilogue (oracle.swiglu, oracle.swiglu_tolerance).

h = silu(g) * u with silu(g) = g / (1 + exp(-g)), the activation of the gated MLP of the
models the pages evaluate.  Pinned by closed-form values (the constant e), the identity
silu(g) - silu(-g) = g, limits, a pure-Python evaluation through math.exp, the slope
bound the tolerance relies on, and a composition check against the pinned matvec
oracle.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth


def test_closed_form_values():
    e = math.e
    assert oracle.swiglu(0.0, 5.0) == 0.0
    assert abs(oracle.swiglu(1.0, 1.0) - 1.0 / (1.0 + 1.0 / e)) < 1e-16
    assert abs(oracle.swiglu(-1.0, 1.0) - (-1.0 / (1.0 + e))) < 1e-16
    assert abs(oracle.swiglu(2.0, -3.0) - (-6.0 / (1.0 + e ** -2))) < 1e-15


def test_odd_part_identity_and_limits():
    g = np.linspace(-30, 30, 2001)
    assert np.allclose(oracle.swiglu(g, 1.0) - oracle.swiglu(-g, 1.0), g, rtol=0, atol=1e-13)
    assert abs(oracle.swiglu(60.0, 1.0) - 60.0) < 1e-20
    assert abs(oracle.swiglu(-60.0, 1.0)) < 1e-20
    assert oracle.swiglu(-1000.0, 1.0) == 0.0  # exp overflow handled


def test_against_pure_python():
    g = synth.rng(5).normal(0, 4, 200)
    u = synth.rng(6).normal(0, 1, 200)
    ref = [gi / (1 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    assert np.allclose(oracle.swiglu(g, u), ref, rtol=1e-15, atol=0)


def test_slope_bound():
    """sup |silu'| (attained near g = 2.4) is below the constant the tolerance uses."""
    g = np.linspace(-20, 20, 400001)
    s = 1 / (1 + np.exp(-g))
    d = s * (1 + g * (1 - s))
    assert 1.09 < d.max() <= oracle.SILU_SLOPE_BOUND
    assert d.min() >= -oracle.SILU_SLOPE_BOUND


def test_tolerance_covers_perturbed_inputs():
    """Inputs moved by their full matvec tolerance stay inside the derived bound."""
    r = synth.rng(9)
    g, u = r.normal(0, 3, 5000), r.normal(0, 3, 5000)
    ag, au = np.abs(g) + r.uniform(0, 5, 5000), np.abs(u) + r.uniform(0, 5, 5000)
    eg, eu = 1e-2 * np.abs(g) + 1e-3 * ag, 1e-2 * np.abs(u) + 1e-3 * au
    tol = oracle.swiglu_tolerance(g, ag, u, au)
    h = oracle.swiglu(g, u)
    for sg in (-1, 1):
        for su in (-1, 1):
            hp = oracle.swiglu(g + sg * eg, u + su * eu)
            assert (np.abs(hp - h) <= tol).all()


def test_composition_with_matvec_oracle():
    R, K = 24, 256
    Wg, Wu = synth.weights(R, K, 1, 1), synth.weights(R, K, 1, 2)
    n = oracle.col_norm(synth.calib_acts(K, 1))
    (gm, gv), (um, uv) = oracle.prune_pack(Wg, n, 2, 4), oracle.prune_pack(Wu, n, 2, 4)
    x = synth.decode_x(2, K, 1)
    g, _ = oracle.spmv(gm, gv, x, K)
    u, _ = oracle.spmv(um, uv, x, K)
    h = oracle.swiglu(g, u)
    assert h.shape == (2, R)
    assert np.allclose(h, g * u / (1 + np.exp(-g)), rtol=1e-15, atol=0)
