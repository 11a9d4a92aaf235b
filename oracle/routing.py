"""MoE routing -> contiguous grouped-GEMM layout, as the oracle defines it.

TEST INFRASTRUCTURE ONLY (see oracle/e4m3.py for who may import this).

The contiguous layout of DeepGEMM's MoE grouped GEMM (release news,
ctol-kr.com, section 4; DeepGEMM explainer, opsoai.com, MoE section) stacks
the rows routed to each expert one expert after another, each expert's run
padded to a multiple of the 128-row M block, and names the expert of every
128-row block.  The pages describe the layout, not the step that builds it
from the router's top-k choices; that step is written here in its plainest
form.

Readings of points the pages leave open:
  * experts appear in id order 0 .. E-1; inside an expert, its tokens appear
    in ascending token order (a stable, deterministic order);
  * a token routed to the same expert twice (a repeated id in its top-k row)
    contributes one row; ids outside [0, E) route nowhere;
  * padding rows hold zeros, which quantize to code 0 with scale 1;
  * the buffers have a fixed capacity of m_cap rows; the 128-row blocks past
    the last expert's run carry the expert id -1 and hold padding.
"""
from __future__ import annotations

import numpy as np

from .scaling import GROUP, quantize_1x128


def contiguous_layout(topk_ids, num_experts: int, m_cap: int):
    """topk_ids int [T, k] -> (row_token int32 [m_cap] (-1 = padding),
    block_expert int32 [m_cap/128] (-1 past the last run), offsets int32
    [E + 1] (first row of each expert's run; offsets[E] = rows in use),
    counts int32 [E])."""
    ids = np.asarray(topk_ids)
    T = ids.shape[0]
    assert m_cap % GROUP == 0
    row_token = np.full(m_cap, -1, np.int32)
    block_expert = np.full(m_cap // GROUP, -1, np.int32)
    offsets = np.zeros(num_experts + 1, np.int32)
    counts = np.zeros(num_experts, np.int32)
    row = 0
    for e in range(num_experts):
        offsets[e] = row
        toks = [t for t in range(T) if (ids[t] == e).any()]
        counts[e] = len(toks)
        padded = -(-len(toks) // GROUP) * GROUP
        assert row + padded <= m_cap, "capacity too small"
        row_token[row:row + len(toks)] = toks
        block_expert[row // GROUP:(row + padded) // GROUP] = e
        row += padded
    offsets[num_experts] = row
    return row_token, block_expert, offsets, counts


def token_rows(topk_ids, num_experts: int, m_cap: int):
    """The inverse of the layout's row map: int32 [T, k] whose entry (t, j) is
    the row holding token t's copy for its j-th expert id, or -1 where that id
    routes nowhere (outside [0, E)) or repeats an earlier id of the same
    token (the token has one row per distinct expert).  This is the map the
    step after the second expert GEMM needs to bring each token's k rows
    back; it is read off the layout defined above."""
    ids = np.asarray(topk_ids)
    row_token, block_expert, _, _ = contiguous_layout(ids, num_experts, m_cap)
    out = np.full(ids.shape, -1, np.int32)
    for r in range(m_cap):
        t = int(row_token[r])
        if t < 0:
            continue
        e = int(block_expert[r // GROUP])
        j = int(np.nonzero(ids[t] == e)[0][0])     # the first position holding e
        out[t, j] = r
    return out


def gather_quantize(x, row_token):
    """Rows x[row_token[r]] (zeros where row_token[r] < 0) quantized 1x128:
    (q uint8 [m_cap, H], s float32 [H/128, m_cap])."""
    x = np.asarray(x, dtype=np.float32)
    rt = np.asarray(row_token)
    g = np.zeros((rt.shape[0], x.shape[1]), np.float32)
    live = rt >= 0
    g[live] = x[rt[live]]
    return quantize_1x128(g)


def capacity(tokens: int, topk: int, num_experts: int) -> int:
    """Smallest m_cap that holds any routing of `tokens` tokens with `topk`
    choices each: every routed row plus up to 127 padding rows per expert,
    rounded up to whole 128-row blocks."""
    return -(-(tokens * topk + num_experts * (GROUP - 1)) // GROUP) * GROUP
