"""FP64 GEMMs on dequantized e4m3 operands: the plain definition the HIP path
must reach.

TEST INFRASTRUCTURE ONLY (see oracle/e4m3.py for who may import this).

The method multiplies FP8 operands and returns an FP32 result (cuda-deepseek
blog, hrletsgo.me, list item 5).  DeepGEMM reaches that result by letting the
tensor cores form FP8 partial sums and promoting them at a fixed interval into
FP32 accumulators on the CUDA cores, where the fine-grained scales are applied
(DeepGEMM release news, ctol-kr.com, section 1 "FP8": two-level accumulation).
Two-level accumulation is an evaluation order of one sum, so the oracle is the
sum itself, over dequantized operands, in float64:

    A[m,k] = e4m3(qa[m,k]) * sa[k // 128, m]
    B[n,k] = e4m3(qb[n,k]) * sb[n // 128, k // 128]
    C[m,n] = sum_k A[m,k] * B[n,k]
    S[m,n] = sum_k |A[m,k] * B[n,k]|         (tolerance base)

Every dequantized value is exact in float64 (4 + 24 significant bits).
The grouped forms are the MoE grouped GEMM in its contiguous and masked
layouts (DeepGEMM explainer, opsoai.com, MoE section; release news section 4
"MoE"): each row block, or each expert's valid rows, is a dense product with
that expert's weights.  MXFP8 (aitrends.kr, MXFP8 section and glossary) scales
each 32-element block by 2**(byte - 127).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import decode
from .scaling import GROUP, MX_BLOCK, e8m0_value


def dequant_1x128(q, s):
    """q uint8 [rows, K], s float32 [K/128, rows] -> float64 [rows, K]."""
    q = np.asarray(q)
    rows, K = q.shape
    s64 = np.asarray(s, dtype=np.float64)
    assert s64.shape == (K // GROUP, rows)
    return decode(q) * np.repeat(s64.T, GROUP, axis=1)


def dequant_128x128(q, s):
    """q uint8 [N, K], s float32 [ceil(N/128), K/128] -> float64 [N, K]."""
    q = np.asarray(q)
    N, K = q.shape
    s64 = np.asarray(s, dtype=np.float64)
    assert s64.shape == (-(-N // GROUP), K // GROUP)
    full = np.repeat(np.repeat(s64, GROUP, axis=0)[:N], GROUP, axis=1)
    return decode(q) * full


def dequant_mx(q, e):
    """q uint8 [rows, K], e uint8 [rows, K/32] -> float64 [rows, K]."""
    q = np.asarray(q)
    return decode(q) * np.repeat(e8m0_value(e), MX_BLOCK, axis=-1)


def matmul_with_base(A, B):
    """C = A @ B^T and S = |A| @ |B|^T in float64."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    return A @ B.T, np.abs(A) @ np.abs(B).T


def gemm_blockscaled(qa, sa, qb, sb):
    """Dense block-scaled GEMM.  qa [M,K], sa [K/128,M], qb [N,K],
    sb [ceil(N/128),K/128] -> (C [M,N], S [M,N]) in float64."""
    return matmul_with_base(dequant_1x128(qa, sa), dequant_128x128(qb, sb))


def grouped_contiguous(qa, sa, qb, sb, block_expert):
    """Contiguous-layout grouped GEMM.  The rows of all experts are stacked in
    qa [M_total, K] (M_total a multiple of 128); block_expert[i] names the
    expert of rows [128 i, 128 i + 128).  qb [E, N, K], sb [E, ceil(N/128), K/128].
    Returns (C, S), each [M_total, N]."""
    qa = np.asarray(qa)
    M, K = qa.shape
    E, N, _ = qb.shape
    be = np.asarray(block_expert)
    assert M % GROUP == 0 and be.shape == (M // GROUP,)
    A = dequant_1x128(qa, sa)
    C = np.zeros((M, N))
    S = np.zeros((M, N))
    for e in range(E):
        rows = np.repeat(be == e, GROUP)
        if rows.any():
            C[rows], S[rows] = matmul_with_base(A[rows], dequant_128x128(qb[e], sb[e]))
    return C, S


def grouped_masked(qa, sa, qb, sb, valid):
    """Masked-layout grouped GEMM.  qa [E, cap, K], sa [E, K/128, cap],
    qb [E, N, K], sb [E, ceil(N/128), K/128], valid [E] in [0, cap].
    Returns (C, S) [E, cap, N]; rows at or past valid[e] are NaN, meaning
    "not defined: the kernel must leave them untouched"."""
    E, cap, K = qa.shape
    N = qb.shape[1]
    C = np.full((E, cap, N), np.nan)
    S = np.full((E, cap, N), np.nan)
    for e in range(E):
        v = int(valid[e])
        if v:
            A = dequant_1x128(qa[e], sa[e])[:v]
            C[e, :v], S[e, :v] = matmul_with_base(A, dequant_128x128(qb[e], sb[e]))
    return C, S


def gemm_mx(qa, ea, qb, eb, valid=None):
    """MXFP8 grouped GEMM.  qa [G, M, K], ea [G, M, K/32], qb [G, N, K],
    eb [G, N, K/32], valid None (every row) or [G] in [0, M].
    Returns (C, S) [G, M, N]; rows at or past valid[g] are NaN."""
    G, M, K = qa.shape
    N = qb.shape[1]
    C = np.full((G, M, N), np.nan)
    S = np.full((G, M, N), np.nan)
    for g in range(G):
        v = M if valid is None else int(valid[g])
        if v:
            A = dequant_mx(qa[g][:v], ea[g][:v])
            C[g, :v], S[g, :v] = matmul_with_base(A, dequant_mx(qb[g], eb[g]))
    return C, S


def grouped_contiguous_mx(qa, ea, qb, eb, block_expert):
    """Contiguous-layout grouped GEMM with MXFP8 operands (aitrends.kr B200
    article, MXFP8 section: MXFP8 grouped GEMM for the MoE experts; layout as
    grouped_contiguous).  qa [M_total, K], ea [M_total, K/32], qb [E, N, K],
    eb [E, N, K/32]; block_expert[i] names the expert of rows [128 i, 128 i +
    128).  Returns (C, S), each [M_total, N]; blocks whose expert id is
    outside [0, E) are left NaN (undefined)."""
    qa = np.asarray(qa)
    M, K = qa.shape
    E, N, _ = qb.shape
    be = np.asarray(block_expert)
    assert M % GROUP == 0 and be.shape == (M // GROUP,)
    A = dequant_mx(qa, ea)
    C = np.full((M, N), np.nan)
    S = np.full((M, N), np.nan)
    for e in range(E):
        rows = np.repeat(be == e, GROUP)
        if rows.any():
            C[rows], S[rows] = matmul_with_base(A[rows], dequant_mx(qb[e], eb[e]))
    return C, S


def round_to_bf16(c) -> np.ndarray:
    """float64 -> nearest bfloat16 (8 significant bits), ties to even, as the
    float32 value that bfloat16 holds.  Finite inputs within bfloat16 range."""
    c = np.asarray(c, dtype=np.float64)
    a = np.abs(c)
    _, e = np.frexp(a)
    binade = np.maximum(e - 1, -126)
    quantum = np.ldexp(1.0, binade - 7)
    v = np.rint(a / quantum) * quantum
    return np.where(np.signbit(c), -v, v).astype(np.float32)
