"""OCP FP8 E4M3 ("e4m3fn") codec, written from the format's definition.

TEST INFRASTRUCTURE ONLY.  This package is the CPU oracle that the HIP path is
checked against.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import it; the product library never
does, and it shares no code, table or constant generator with the HIP kernels.

Which FP8 the method uses.  The pages only say "FP8": the DeepGEMM explainer
(opsoai.com, DeepGEMM post, opening section) and the DeepGEMM release news
(ctol-kr.com, section 1 "FP8") name the format without its layout, and the
cuda-deepseek blog demo (hrletsgo.me) stands FP8 in with a signed char clamped
to +-127, which is not an FP8 format at all.  We take the reading the rest of
the method supports: OCP E4M3 with no infinities (sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent 15 with mantissa 7 is NaN; largest
finite value 1.75 * 2**8 = 448), encoded by round-to-nearest-even and
saturated to +-448, with the sign of zero kept.

Every value here is computed exactly in float64: e4m3 values have 4
significant bits and every quantity the encoder forms is a float32 value
times a power of two.
"""
from __future__ import annotations

import math

import numpy as np

EXPONENT_BIAS = 7
MANTISSA_BITS = 3
MAX_FINITE = 448.0          # 1.75 * 2**8, the largest finite e4m3 value
MIN_NORMAL_EXP = -6         # exponent field 1 means 2**(1 - 7)
NAN_CODES = (0x7F, 0xFF)


def decode_code(code: int) -> float:
    """Value of one 8-bit e4m3 code (closed form of the format)."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return math.nan
    if exp_field == 0:                       # subnormal: m * 2**-9
        return sign * mant * 2.0 ** (MIN_NORMAL_EXP - MANTISSA_BITS)
    return sign * 2.0 ** (exp_field - EXPONENT_BIAS) * (1.0 + mant / 8.0)


DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(q) -> np.ndarray:
    """e4m3 codes (uint8 array) -> exact float64 values (NaN for 0x7F/0xFF)."""
    return DECODE_TABLE[np.asarray(q, dtype=np.uint8)]


def round_to_e4m3_value(y) -> np.ndarray:
    """Round finite values to the nearest e4m3 magnitude, ties to even, then
    saturate at 448.  Returns float64 values carrying the input's sign.

    Inside one binade [2**E, 2**(E+1)) the e4m3 values are the multiples of the
    quantum 2**(E-3); below 2**-6 the subnormals are the multiples of 2**-9,
    i.e. the same quantum as the lowest normal binade.  Rounding a magnitude to
    the nearest multiple of its quantum with ties to the even multiple is
    exactly round-to-nearest-even on the 3-bit mantissa (an even multiple has
    an even mantissa, and a carry into the next binade lands on an e4m3 value).
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("e4m3 encode: inputs must be finite")
    a = np.abs(y)
    _, e = np.frexp(a)                       # a = f * 2**e with f in [0.5, 1)
    binade = np.maximum(e - 1, MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, binade - MANTISSA_BITS)
    v = np.rint(a / quantum) * quantum       # np.rint rounds half to even
    v = np.minimum(v, MAX_FINITE)            # saturate instead of overflowing
    return np.where(np.signbit(y), -v, v)


def encode(y) -> np.ndarray:
    """Finite float values -> e4m3 codes (uint8), RNE with saturation."""
    v = round_to_e4m3_value(y)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** MIN_NORMAL_EXP
    # subnormals and zero: the code is the count of 2**-9 quanta
    code[sub] = (a[sub] * 2.0 ** (MANTISSA_BITS - MIN_NORMAL_EXP)).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        f, e = np.frexp(a[nrm])              # a = (2f) * 2**(e-1), 2f in [1, 2)
        exp_field = (e - 1) + EXPONENT_BIAS
        mant = ((2.0 * f - 1.0) * 8.0).astype(np.int64)
        code[nrm] = (exp_field << MANTISSA_BITS) | mant
    return (code.astype(np.uint8) | sign).astype(np.uint8)
