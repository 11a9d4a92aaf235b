"""The two training-backward pieces of a grouped (MoE) linear layer, as the
oracle defines them.

TEST INFRASTRUCTURE ONLY (see oracle/e4m3.py for who may import this).

The pages say that in real training the gradients are computed in the same
FP8 / FP32 mixed precision as the forward pass, with the details left out of
the demo (cuda-deepseek blog, hrletsgo.me, backward-pass step of the training
loop), and that the MoE experts of DeepSeek-V3 train with FP8 grouped GEMMs
(aitrends.kr B200 article, MXFP8 section).  The weight gradient of expert e
is dW_e = dY_e^T X_e, a sum over the tokens routed to e; in the contiguous
layout those tokens are the rows offsets[e] .. offsets[e+1] - 1 (whole
128-row blocks).  Readings of what the pages leave open:

  * both operands of the weight gradient are laid out with the token axis
    contiguous (A := dY^T [N][T], B := X^T [H][T]) and quantized 1x128 along
    that axis: "1x128 along the other axis" of the row-major tensors;
  * the K-grouped GEMM multiplies, for each group g, the K range
    offsets[g] .. offsets[g+1] of A and B, with one FP32 scale per row and
    128-wide K block on both operands:
        D_g[m, n] = sum_{k in group g} A[m, k] * B[n, k];
    an empty group gives zeros.

Everything is float64 on dequantized values, as for the forward GEMMs.
"""
from __future__ import annotations

import numpy as np

from .gemm import dequant_1x128, matmul_with_base
from .scaling import GROUP, quantize_1x128


def quantize_1x128_transposed(x):
    """x [rows, cols] (rows % 128 == 0) -> the 1x128 quantization of x^T:
    (q uint8 [cols, rows], s float32 [rows/128, cols])."""
    x = np.asarray(x)
    assert x.shape[0] % GROUP == 0, "the grouped axis must hold whole groups"
    return quantize_1x128(np.ascontiguousarray(x.T))


def grouped_k(qa, sa, qb, sb, offsets):
    """qa [M, K] with sa [K/128, M], qb [N, K] with sb [K/128, N] (1x128 on
    both), offsets [G + 1] K offsets (multiples of 128, non-decreasing) ->
    (C [G, M, N], S [G, M, N]) in float64."""
    A = dequant_1x128(qa, sa)
    B = dequant_1x128(qb, sb)
    off = np.asarray(offsets, np.int64)
    G = off.shape[0] - 1
    M, N = A.shape[0], B.shape[0]
    C = np.zeros((G, M, N))
    S = np.zeros((G, M, N))
    for g in range(G):
        k0, k1 = int(off[g]), int(off[g + 1])
        assert k0 % GROUP == 0 and k1 % GROUP == 0 and k0 <= k1
        if k1 > k0:
            C[g], S[g] = matmul_with_base(A[:, k0:k1], B[:, k0:k1])
    return C, S
