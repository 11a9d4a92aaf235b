"""Seeded synthetic inputs for the fine-grained FP8 GEMM workloads.

This module is shared by the tests and the benchmark.  It holds no
arithmetic of the method (no scaling, no quantization, no GEMM, no routing
layout): only FP32 source tensors, the router's top-k expert ids and the
masked layout's counts.  Every draw uses numpy's PCG64 generator seeded with
[workload id, stream], stream 0 = A, 1 = B, 2 = row modifiers, 3 = routing
or counts, 4 = second weight set, 5 = second activation set.

Workloads (shapes from the DeepGEMM explainer, opsoai.com, speed-up table:
64x2112x7168, 64x24576x1536, 128x7168x2048; MoE grouped GEMM in contiguous and
masked layouts from the DeepGEMM release news, ctol-kr.com, section 4):
  0  tiny dense: A, B ~ N(0,1), max(1, round(0.01 M)) rows of A times 100
  1  skinny dense: A = z * r_m with ln r_m ~ U(ln 0.01, ln 10); B ~ N(0, 1/K)
  2  prefill dense: A = z * |t_m| with t_m ~ Student-t(3) per row; B ~ N(0, 1/K)
  3  MoE contiguous: tokens pick top-k distinct experts with Zipf(1.1)
     popularity (the layout itself is the routing step's output)
  4  MoE masked: per-expert valid counts ~ U{0..cap}; rows past the count are
     junk (finite here; tests poison the quantized copies)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

def rng(workload: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([workload, stream])


def _normal(g: np.random.Generator, shape, std=1.0) -> np.ndarray:
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def dense_a(workload: int, M: int, K: int, kind: str) -> np.ndarray:
    """Activation matrix A [M, K] float32 with the row structure of `kind`."""
    z = _normal(rng(workload, 0), (M, K))
    g = rng(workload, 2)
    if kind == "outlier_rows":
        n_out = max(1, int(round(0.01 * M)))
        rows = g.choice(M, size=n_out, replace=False)
        z[rows] *= np.float32(100.0)
    elif kind == "lognormal_rows":
        r = np.exp(g.uniform(np.log(0.01), np.log(10.0), size=M)).astype(np.float32)
        z *= r[:, None]
    elif kind == "t3_rows":
        t = np.abs(g.standard_t(3, size=M)).astype(np.float32)
        z *= t[:, None]
    elif kind == "t3_elements":
        z = g.standard_t(3, size=(M, K)).astype(np.float32)
    elif kind != "normal":
        raise ValueError(kind)
    return z


def dense_b(workload: int, N: int, K: int, unit_variance: bool = False,
            stream: int = 1) -> np.ndarray:
    """Weight matrix B [N, K] float32 (a Linear weight [out][in]); N(0, 1/K)
    unless unit_variance."""
    return _normal(rng(workload, stream), (N, K), 1.0 if unit_variance else K ** -0.5)


@dataclass
class DenseCase:
    name: str
    workload: int
    M: int
    N: int
    K: int
    a_kind: str
    b_unit: bool


DENSE_CASES = {
    "tiny": DenseCase("tiny 64x256x512", 0, 64, 256, 512, "outlier_rows", True),
    "skinny_a": DenseCase("skinny 64x2112x7168", 1, 64, 2112, 7168, "lognormal_rows", False),
    "skinny_b": DenseCase("skinny 64x24576x1536", 1, 64, 24576, 1536, "lognormal_rows", False),
    "prefill_a": DenseCase("prefill 128x7168x2048", 2, 128, 7168, 2048, "t3_rows", False),
    "prefill_b": DenseCase("prefill 4096x7168x2048", 2, 4096, 7168, 2048, "t3_rows", False),
}


def dense_case(name: str, M=None, N=None, K=None):
    """(A, B) float32 for a named dense case; M/N/K override the size only."""
    c = DENSE_CASES[name]
    M, N, K = M or c.M, N or c.N, K or c.K
    return dense_a(c.workload, M, K, c.a_kind), dense_b(c.workload, N, K, c.b_unit)


# ----------------------------------------------------------------- MoE routing
def zipf_topk_routing(workload: int, tokens: int, experts: int, topk: int,
                      s: float = 1.1) -> np.ndarray:
    """[tokens, topk] int32 distinct experts per token, drawn without
    replacement with probability proportional to (e + 1)^-s (Gumbel top-k on
    the log-probabilities)."""
    g = rng(workload, 3)
    logp = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    keys = logp[None, :] + g.gumbel(size=(tokens, experts))
    return np.argsort(-keys, axis=1)[:, :topk].astype(np.int32)


@dataclass
class ContiguousCase:
    tokens: int = 8192
    hidden: int = 7168       # K of the first expert GEMM, N of the second
    inter: int = 4096        # N of the first expert GEMM
    inter2: int = 2048       # K of the second expert GEMM
    experts: int = 32
    topk: int = 8
    workload: int = 3


def contiguous_sources(c: ContiguousCase):
    """The FP32 sources of the contiguous MoE workload: (topk ids [tokens,
    topk] int32, token rows x [tokens, hidden], W1 [E, inter, hidden],
    W2 [E, hidden, inter2]).  The row layout the grouped GEMM consumes is
    built from the ids by the method's routing step, not here."""
    ids = zipf_topk_routing(c.workload, c.tokens, c.experts, c.topk)
    x = _normal(rng(c.workload, 0), (c.tokens, c.hidden))
    w1 = _normal(rng(c.workload, 1), (c.experts, c.inter, c.hidden), c.hidden ** -0.5)
    w2 = _normal(rng(c.workload, 4), (c.experts, c.hidden, c.inter2), c.inter2 ** -0.5)
    return ids, x, w1, w2


def contiguous_a2(c: ContiguousCase, rows: int):
    """The second expert GEMM's FP32 input, N(0, 1), one row per layout row
    (the caller zeroes the padding rows)."""
    return _normal(rng(c.workload, 5), (rows, c.inter2))


@dataclass
class MaskedCase:
    experts: int = 16
    cap: int = 256
    N: int = 4096
    K: int = 7168
    workload: int = 4


def masked_case_counts(c: MaskedCase) -> np.ndarray:
    """Per-expert valid counts ~ U{0..cap} (inclusive), int32 [E]."""
    return rng(c.workload, 3).integers(0, c.cap, size=c.experts, endpoint=True).astype(np.int32)


def masked_case(c: MaskedCase):
    """(valid [E] int32 in [0, cap], A [E, cap, K], B [E, N, K]).  Rows of A at
    or past valid[e] hold large finite junk."""
    valid = masked_case_counts(c)
    a = _normal(rng(c.workload, 0), (c.experts, c.cap, c.K))
    junk = rng(c.workload, 2)
    for e in range(c.experts):
        v = int(valid[e])
        if v < c.cap:
            a[e, v:] = junk.uniform(-1e30, 1e30, size=(c.cap - v, c.K)).astype(np.float32)
    b = _normal(rng(c.workload, 1), (c.experts, c.N, c.K), c.K ** -0.5)
    return valid, a, b
