"""Gated activation between the two expert GEMMs of an MoE layer, as the
oracle defines it.

TEST INFRASTRUCTURE ONLY (see oracle/e4m3.py for who may import this).

The pages describe the expert layer as quantize -> grouped GEMM -> restore
(aitrends.kr B200 article, MXFP8 pipeline diagram) and give the widths of the
two expert weights (W1 maps the hidden size to twice the input width of W2),
but they never name the activation between them.  The plainest reading that
fits a first GEMM twice as wide as the second one's input is a gated linear
unit: half of W1's outputs gate the other half.  The gate used here is SiLU,
x * sigmoid(x) (the SwiGLU form of DeepSeek-style expert MLPs); this is a
reading, not something the pages state.

Layout (a free choice, fixed in fg8.h and written out here on its own): the
rows of W1 interleave in 128-row blocks, gate block j at rows 256 j .. 256 j
+ 127 and up block j at rows 256 j + 128 .. 256 j + 255, so output column
block j of the activation h reads columns 256 j .. 256 j + 255 of the W1
product: h[:, 128 j + c] = silu(C[:, 256 j + c]) * C[:, 256 j + 128 + c].

Everything is float64.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def silu(x):
    """x * sigmoid(x) = x / (1 + e^-x), float64; -0.0 for very negative x."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu_interleaved(C):
    """C [M, N] (N % 256 == 0), the product with the interleaved W1 ->
    h [M, N/2] = silu(gate) * up, block by block as in the module text."""
    C = np.asarray(C, np.float64)
    M, N = C.shape
    assert N % (2 * GROUP) == 0, "N must hold whole gate/up block pairs"
    blocks = C.reshape(M, N // (2 * GROUP), 2, GROUP)
    gate, up = blocks[:, :, 0, :], blocks[:, :, 1, :]
    return (silu(gate) * up).reshape(M, N // 2)


def gate_up_of(C):
    """The (gate, up) halves of C [M, N] in h's column order, each [M, N/2]."""
    C = np.asarray(C)
    M, N = C.shape
    blocks = C.reshape(M, N // (2 * GROUP), 2, GROUP)
    return (blocks[:, :, 0, :].reshape(M, N // 2), blocks[:, :, 1, :].reshape(M, N // 2))
