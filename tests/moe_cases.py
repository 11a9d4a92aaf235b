"""The contiguous MoE workload as the tests feed it to the grouped GEMMs: the
seeded sources of tests/inputs.py laid out by the oracle's routing step
(oracle/routing.py), trimmed to the rows in use."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import inputs
from oracle import routing


@dataclass
class Layout:
    """Rows of all experts stacked, each expert padded to a multiple of 128."""
    row_token: np.ndarray      # [m_total] int32, source token of each row, -1 = padding
    block_expert: np.ndarray   # [m_total / 128] int32, expert of each 128-row block
    counts: np.ndarray         # [E] int32 routed rows per expert (before padding)
    offsets: np.ndarray        # [E + 1] int32 first row of each expert's run

    @property
    def m_total(self) -> int:
        return int(self.row_token.shape[0])

    @property
    def valid_rows(self) -> int:
        return int(self.counts.sum())


def contiguous_layout(ids, experts: int) -> Layout:
    """The oracle's contiguous layout of the top-k ids, without the spare
    capacity past the last expert's run."""
    ids = np.asarray(ids)
    cap = routing.capacity(ids.shape[0], ids.shape[1], experts)
    rt, be, off, cnt = routing.contiguous_layout(ids, experts, cap)
    used = int(off[experts])
    return Layout(rt[:used], be[:used // 128], cnt, off)


def gather_rows(x, row_token):
    """x[row_token] with zero rows for padding (-1)."""
    out = np.zeros((row_token.shape[0], x.shape[1]), dtype=x.dtype)
    live = row_token >= 0
    out[live] = x[row_token[live]]
    return out


def contiguous_case(c: inputs.ContiguousCase):
    """Inputs of both expert GEMMs in the contiguous layout:
    (layout, A1 [m_total, hidden], W1 [E, inter, hidden], A2 [m_total, inter2],
    W2 [E, hidden, inter2]); padding rows of A1 and A2 are zero."""
    ids, x, w1, w2 = inputs.contiguous_sources(c)
    lay = contiguous_layout(ids, c.experts)
    a1 = gather_rows(x, lay.row_token)
    del x
    a2 = inputs.contiguous_a2(c, lay.m_total)
    a2[lay.row_token < 0] = 0.0
    return lay, a1, w1, a2, w2
