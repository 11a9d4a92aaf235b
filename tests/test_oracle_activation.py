"""Pins of oracle/activation.py against closed forms of SiLU and a
hand-built interleaved product (no GPU)."""
import math

import numpy as np

from oracle import activation


def test_silu_closed_forms():
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4 exactly
    assert math.isclose(activation.silu(math.log(3.0)), 0.75 * math.log(3.0), rel_tol=1e-15)
    assert activation.silu(0.0) == 0.0
    # sigmoid(x) + sigmoid(-x) = 1, so silu(x) - silu(-x) = x
    x = np.random.default_rng(5).standard_normal(1000) * 8
    assert np.allclose(activation.silu(x) - activation.silu(-x), x, rtol=0, atol=1e-13)
    # the tails: silu(x) -> x above, -> -|x| e^-|x| below
    assert math.isclose(activation.silu(40.0), 40.0, rel_tol=1e-15)
    assert math.isclose(activation.silu(-40.0), -40.0 * math.exp(-40.0), rel_tol=1e-12)
    assert activation.silu(-1000.0) == 0.0 and math.copysign(1, activation.silu(-1000.0)) < 0
    # slope bound used by the tolerance of the fused GPU epilogue: |silu'| < 1.1
    t = np.linspace(-30, 30, 600001)
    d = np.diff(activation.silu(t)) / np.diff(t)
    assert np.abs(d).max() < 1.1 and np.abs(d).max() > 1.09


def test_interleaved_blocks_pair_gate_with_their_own_up():
    M, N = 3, 512
    C = np.zeros((M, N))
    ln3 = math.log(3.0)
    C[:, 0:128] = ln3          # gate block 0
    C[:, 128:256] = 2.0        # up block 0
    C[:, 256:384] = 0.0        # gate block 1: silu(0) = 0
    C[:, 384:512] = 7.0        # up block 1
    C[1, 5] = -ln3             # one gate entry: silu(-ln 3) = -ln3 / 4
    h = activation.swiglu_interleaved(C)
    assert h.shape == (M, 256)
    assert np.allclose(h[:, :128][[0, 2]], 1.5 * ln3, rtol=1e-15)
    assert math.isclose(h[1, 5], -0.25 * ln3 * 2.0, rel_tol=1e-15)
    assert np.all(h[:, 128:] == 0.0)
    g, u = activation.gate_up_of(C)
    assert np.all(u[:, :128] == 2.0) and np.all(g[:, 128:] == 0.0) and np.all(u[:, 128:] == 7.0)

