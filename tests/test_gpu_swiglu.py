"""The contiguous W1 GEMM with the SiLU-gated activation and the 1x128
quantization of its output fused into the epilogue, against the oracle's
product and activation (oracle/gemm.py, oracle/activation.py).  Codes and
scales are checked against the bounds of tests/parity.py."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
import inputs
import moe_cases
from oracle import scaling
from parity import check_swiglu_quant, ref_blockscaled

pytestmark = pytest.mark.gpu


def _gpu(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in arrays]


def _case(tokens, hidden, inter, experts, topk, workload=33):
    c = inputs.ContiguousCase(tokens=tokens, hidden=hidden, inter=inter, inter2=256,
                              experts=experts, topk=topk, workload=workload)
    lay, a1, w1, _, _ = moe_cases.contiguous_case(c)
    return c, lay, a1, w1


@pytest.mark.parametrize("shape", [(300, 512, 512, 6, 2), (700, 1024, 768, 9, 3)])
def test_swiglu_small(dev, shape):
    c, lay, a1, w1 = _case(*shape)
    print(f"swiglu small {shape}", flush=True)
    qa, sa = scaling.quantize_1x128(a1)
    qb, sb = scaling.quantize_128x128(w1)
    ta, tsa, tb, tsb, tbe = _gpu(qa, sa, qb, sb, lay.block_expert)
    q, s = fg8.grouped_gemm_fp8_contiguous_swiglu(ta, tsa, tb, tsb, tbe)
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    moved = 0
    for e in range(c.experts):
        rows = np.repeat(lay.block_expert == e, 128)
        if not rows.any():
            continue
        C, S, F = ref_blockscaled(qa[rows], sa[:, rows], qb[e], sb[e])
        moved += check_swiglu_quant(q[rows], s[:, rows], C, S, F, c.hidden, f"expert {e}")
    # padding rows of A are zero: h = 0 there, codes 0 and scale 1
    pad = lay.row_token < 0
    assert np.all(q[pad] == 0) and np.all(s[:, pad] == 1.0)
    print(f"codes off the oracle's own rounding of h: {moved} of {q.size}")


def test_swiglu_skips_out_of_range_blocks(dev):
    c, lay, a1, w1 = _case(300, 512, 512, 6, 2)
    be = lay.block_expert.copy()
    be[1] = -1
    be[-1] = c.experts + 3
    qa, sa = scaling.quantize_1x128(a1)
    qb, sb = scaling.quantize_128x128(w1)
    ta, tsa, tb, tsb, tbe = _gpu(qa, sa, qb, sb, be)
    M = a1.shape[0]
    q0 = torch.full((M, 256), 0x5A, dtype=torch.uint8, device="cuda")
    s0 = torch.full((2, M), -7.0, dtype=torch.float32, device="cuda")
    q, s = fg8.grouped_gemm_fp8_contiguous_swiglu(ta, tsa, tb, tsb, tbe, q_out=q0, s_out=s0)
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    for b in (1, len(be) - 1):
        assert np.all(q[b * 128:(b + 1) * 128] == 0x5A)
        assert np.all(s[:, b * 128:(b + 1) * 128] == -7.0)
    live = np.repeat((be >= 0) & (be < c.experts), 128)
    assert not np.any(s[:, live] == -7.0)
    for e in range(c.experts):
        rows = np.repeat(be == e, 128)
        if rows.any():
            C, S, F = ref_blockscaled(qa[rows], sa[:, rows], qb[e], sb[e])
            check_swiglu_quant(q[rows], s[:, rows], C, S, F, c.hidden, f"expert {e}")


def test_swiglu_full_size_every_row(dev):
    """8192 tokens, top-8 of 32 experts (Zipf 1.1), W1 7168 -> 4096 with the
    activation fused: the GPU quantizes and multiplies everything; the oracle
    quantizes the token rows and two gate/up block pairs of every expert
    itself and checks the two 128-column blocks of h they give on every
    routed row of every expert (padding rows: codes 0, scale 1)."""
    c = inputs.ContiguousCase()
    ids, x, w1, _ = inputs.contiguous_sources(c)
    lay = moe_cases.contiguous_layout(ids, c.experts)
    a1 = moe_cases.gather_rows(x, lay.row_token)
    K = a1.shape[1]
    tA, tW = _gpu(a1, w1)
    del a1
    qa, sa = fg8.fp8_quantize(tA, "1x128")
    qb, sb = fg8.fp8_quantize(tW, "128x128")
    del tA, tW
    tbe = torch.from_numpy(lay.block_expert).cuda()
    q, s = fg8.grouped_gemm_fp8_contiguous_swiglu(qa, sa, qb, sb, tbe)
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    del qa, sa, qb, sb
    pad = lay.row_token < 0
    assert np.all(q[pad] == 0) and np.all(s[:, pad] == 1.0)
    qx, sx = scaling.quantize_1x128(x)            # token rows; a layout row holds one
    del x
    g = np.random.default_rng(405)
    N = w1.shape[1]
    hbs = np.sort(g.choice(N // 256, 2, replace=False))
    hcols = np.concatenate([np.arange(j * 128, j * 128 + 128) for j in hbs])
    rows_e = np.repeat(lay.block_expert, 128)
    moved = total = 0
    for e in range(c.experts):
        rows = np.nonzero((rows_e == e) & ~pad)[0]
        if rows.size == 0:
            continue
        tok = lay.row_token[rows]
        Bq = [scaling.quantize_128x128(w1[e, j * 256 + h * 128:j * 256 + h * 128 + 128])
              for j in hbs for h in (0, 1)]
        qb_o = np.concatenate([y for y, _ in Bq])
        sb_o = np.concatenate([z for _, z in Bq])
        C, S, F = ref_blockscaled(qx[tok], sx[:, tok], qb_o, sb_o)
        moved += check_swiglu_quant(q[np.ix_(rows, hcols)], s[np.ix_(hbs, rows)], C, S, F, K,
                                    f"expert {e}")
        total += rows.size * hcols.size
    print(f"gated epilogue, every routed row: {moved} of {total} codes off the oracle's own "
          f"rounding of h", flush=True)
