"""Fine-grained group scaling to e4m3, as the oracle defines it.

TEST INFRASTRUCTURE ONLY (see oracle/e4m3.py for who may import this).

The method: an FP32 tensor is multiplied by a scaling factor and converted to
FP8, the GEMM runs on FP8, and the result comes back in FP32 (cuda-deepseek
blog, hrletsgo.me, list item 5 of the mixed-precision loop).  The blog's demo
uses one scale per tensor but its own comments say real code scales per tile,
and the DeepGEMM explainer (opsoai.com, validation advice) warns that one wide
scale loses small values.  The granularities used here are the DeepGEMM ones:
1x128 groups along K for activations and 128x128 blocks for weights, with the
scale stored as s = amax / 448 and the element quantized as e4m3(x / s).
MXFP8 shares one power-of-two exponent per 32 consecutive elements
(aitrends.kr article on DeepSeek-V3 MoE training on B200, MXFP8 section and
glossary entry; OCP Microscaling specification named in its resources).

Readings of points the pages leave open:
  * s = fl32(amax / 448) and q = e4m3(fl32(x / s)), both correctly rounded
    float32 divisions;
  * an all-zero group gets s = 1.0 (any s reconstructs zeros);
  * a 128x128 block cut short by the end of the rows takes its amax over the
    rows that exist;
  * MX: E = floor(log2 amax) - 8 clamped to [-127, 127] (8 is the exponent of
    the largest e4m3 binade), E = -127 for an all-zero block, stored as the
    byte E + 127; elements are e4m3(x * 2**-E), saturated at 448.
Inputs must be finite.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import MAX_FINITE, encode

GROUP = 128
MX_BLOCK = 32
MX_EMAX_E4M3 = 8           # floor(log2(448))
E8M0_BIAS = 127


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def scale_from_amax(amax) -> np.ndarray:
    """s = fl32(amax / 448), with s = 1 for an all-zero group."""
    amax = _f32(amax)
    s = amax / np.float32(MAX_FINITE)        # float32 / float32: correctly rounded
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_1x128(x):
    """x float32 [..., rows, cols] -> (q uint8 [..., rows, cols],
    s float32 [..., cols/128, rows]).  One scale per row per 128 columns."""
    x = _f32(x)
    *lead, rows, cols = x.shape
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 128")
    g = x.reshape(*lead, rows, cols // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=-1)                    # [..., rows, cols/128]
    s = scale_from_amax(amax)
    y = g / s[..., None]                                 # float32 division
    q = encode(y.astype(np.float64)).reshape(x.shape)
    return q, np.ascontiguousarray(np.swapaxes(s, -1, -2))


def quantize_128x128(w):
    """w float32 [..., rows, cols] -> (q uint8 [..., rows, cols],
    s float32 [..., ceil(rows/128), cols/128]).  One scale per 128x128 block;
    a block cut by the end of the rows covers only the rows that exist."""
    w = _f32(w)
    *lead, rows, cols = w.shape
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 128")
    nrb = -(-rows // GROUP)
    q = np.empty(w.shape, dtype=np.uint8)
    s = np.empty((*lead, nrb, cols // GROUP), dtype=np.float32)
    for rb in range(nrb):
        r0, r1 = rb * GROUP, min(rows, (rb + 1) * GROUP)
        blk = w[..., r0:r1, :].reshape(*lead, r1 - r0, cols // GROUP, GROUP)
        amax = np.max(np.abs(blk), axis=(-3, -1))        # [..., cols/128]
        sb = scale_from_amax(amax)
        s[..., rb, :] = sb
        y = blk / sb[..., None, :, None]
        q[..., r0:r1, :] = encode(y.astype(np.float64)).reshape(*lead, r1 - r0, cols)
    return q, s


def mx_exponent(amax) -> np.ndarray:
    """Shared exponent E of an MX block from its amax (exact, via frexp)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                    # amax = f * 2**e, f in [0.5, 1)
    E = (e - 1) - MX_EMAX_E4M3               # floor(log2 amax) - 8
    E = np.clip(E, -E8M0_BIAS, E8M0_BIAS)
    return np.where(amax == 0, -E8M0_BIAS, E).astype(np.int64)


def quantize_mx(x):
    """x float32 [..., rows, cols] -> (q uint8 [..., rows, cols],
    e8m0 uint8 [..., rows, cols/32]) with one shared exponent per 32."""
    x = _f32(x)
    *lead, rows, cols = x.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    g = x.reshape(*lead, rows, cols // MX_BLOCK, MX_BLOCK).astype(np.float64)
    E = mx_exponent(np.max(np.abs(g), axis=-1))
    y = np.ldexp(g, -E[..., None])                       # exact power-of-two scaling
    q = encode(y).reshape(x.shape)
    return q, (E + E8M0_BIAS).astype(np.uint8)


def e8m0_value(byte) -> np.ndarray:
    """E8M0 scale byte -> 2**(byte - 127) (0xFF, NaN in the format, is rejected)."""
    b = np.asarray(byte, dtype=np.int64)
    if np.any(b == 0xFF):
        raise ValueError("E8M0 byte 0xFF is NaN")
    return np.ldexp(1.0, b - E8M0_BIAS)
