"""Training-backward pieces on the GPU against the oracle (oracle/backward.py):
the 1x128 quantization along the token axis with transposed codes
(bit-exact), and the K-grouped weight-gradient GEMM (FP32 / BF16 bars of
tests/parity.py)."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
import inputs
from oracle import backward, routing
from parity import TruncRows, check_bf16, check_f32, ref_blockscaled, ref_kgrouped
from test_gpu_quantize import _hard_values

pytestmark = pytest.mark.gpu


def _to_bf16(x):
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("shape", [(1, 128, 64), (2, 384, 192), (1, 1024, 7168)])
def test_transposed_quantize_bit_exact(dev, shape, bf16):
    batch, rows, cols = shape
    g = np.random.default_rng(300 + rows)
    x = np.stack([_hard_values(g, (cols, rows)).T for _ in range(batch)])   # groups down columns
    print(f"transposed quantize {shape} bf16={bf16}", flush=True)
    if bf16:
        bits, x = _to_bf16(np.ascontiguousarray(x))
        t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q, s = fg8.fp8_quantize(t, "1x128_t")
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    assert q.shape == (batch, cols, rows) and s.shape == (batch, rows // 128, cols)
    for b in range(batch):
        qo, so = backward.quantize_1x128_transposed(x[b])
        assert np.array_equal(q[b], qo)
        assert np.array_equal(s[b].view(np.uint32), so.view(np.uint32))


def _operands(T, m, n, seed):
    g = np.random.default_rng(seed)
    dy = (g.standard_normal((T, m)) * np.exp(g.uniform(-3, 3, (T, 1)))).astype(np.float32)
    x = g.standard_normal((T, n)).astype(np.float32)
    qa, sa = backward.quantize_1x128_transposed(dy)
    qb, sb = backward.quantize_1x128_transposed(x)
    return qa, sa, qb, sb


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", [
    (300, 200, [0, 256, 256, 1024, 1152]),          # an empty group, ragged m and n
    (256, 384, [0, 128]),                            # one single-block group
    (64, 130, [0, 512, 1536, 1536, 1536, 2048]),    # trailing empty groups
])
def test_kgrouped_small(dev, case, out_dtype):
    m, n, off = case
    T = off[-1]
    qa, sa, qb, sb = _operands(T, m, n, 310 + m)
    print(f"kgrouped m={m} n={n} offsets={off} out={out_dtype}", flush=True)
    ta, tsa, tb, tsb = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in (qa, sa, qb, sb)]
    toff = torch.tensor(off, dtype=torch.int32, device="cuda")
    d = torch.full((len(off) - 1, m, n), float("nan"), dtype=out_dtype, device="cuda")
    fg8.grouped_gemm_fp8_kgrouped(ta, tsa, tb, tsb, toff, out=d)
    torch.cuda.synchronize()
    C, S, F = ref_kgrouped(qa, sa, qb, sb, off)
    for g in range(len(off) - 1):
        where = f"group {g} K [{off[g]}, {off[g + 1]})"
        if out_dtype == torch.float32:
            got = d[g].cpu().numpy()
            if off[g] == off[g + 1]:
                assert np.all(got == 0.0), where
            check_f32(got, C[g], S[g], max(off[g + 1] - off[g], 128), where, S_flush=F[g])
        else:
            bits = d[g].view(torch.int16).cpu().numpy().view(np.uint16)
            check_bf16(bits, C[g], S[g], max(off[g + 1] - off[g], 128), where, S_flush=F[g])


def test_wgrad_from_the_routing_layout_full_size_sampled(dev):
    """The weight gradient of W1 for the MoE workload (8192 tokens, top-8 of
    32 experts, Zipf 1.1): dY [M_pad, 4096] and X [M_pad, 7168] in the
    contiguous layout (padding rows zero), both quantized along the token
    axis on the GPU, then the K-grouped GEMM over the routing layout's expert
    offsets.  The oracle quantizes the sampled columns itself and checks
    sampled 128 x 128 output blocks of sampled experts."""
    c = inputs.ContiguousCase()
    ids = inputs.zipf_topk_routing(c.workload, c.tokens, c.experts, c.topk)
    m_cap = routing.capacity(c.tokens, c.topk, c.experts)
    rt, be, off, cnt = routing.contiguous_layout(ids, c.experts, m_cap)
    M = int(off[-1])                                    # rows in use
    g = inputs.rng(c.workload, 6)
    dy = g.standard_normal((M, c.inter), dtype=np.float32)
    x = inputs.rng(c.workload, 0).standard_normal((c.tokens, c.hidden), dtype=np.float32)
    X = np.zeros((M, c.hidden), np.float32)
    live = rt[:M] >= 0
    X[live] = x[rt[:M][live]]
    dy[~live] = 0.0
    del x
    tdy = torch.from_numpy(dy).cuda()
    tX = torch.from_numpy(X).cuda()
    qa, sa = fg8.fp8_quantize(tdy, "1x128_t")
    qb, sb = fg8.fp8_quantize(tX, "1x128_t")
    del tdy, tX
    toff = torch.from_numpy(off.astype(np.int32)).cuda()
    d = fg8.grouped_gemm_fp8_kgrouped(qa, sa, qb, sb, toff, out_dtype=torch.float32)
    torch.cuda.synchronize()
    gs = np.random.default_rng(406)
    for e in gs.choice(c.experts, 6, replace=False):
        k0, k1 = int(off[e]), int(off[e + 1])
        if k1 == k0:
            continue
        ib = gs.integers(0, c.inter // 128)
        jb = gs.integers(0, c.hidden // 128)
        rows = np.arange(ib * 128, ib * 128 + 128)
        cols = np.arange(jb * 128, jb * 128 + 128)
        qa_o, sa_o = backward.quantize_1x128_transposed(dy[k0:k1, rows])
        qb_o, sb_o = backward.quantize_1x128_transposed(X[k0:k1, cols])
        C, S, F = ref_kgrouped(qa_o, sa_o, qb_o, sb_o, [0, k1 - k0])
        got = d[e, ib * 128:(ib + 1) * 128, jb * 128:(jb + 1) * 128].cpu().numpy()
        check_f32(got, C[0], S[0], k1 - k0, f"expert {e} block ({ib}, {jb})", S_flush=F[0])


def _dx_rows(qdy, sdy, qw, sw):
    """Oracle dX = dY W for rows of one expert: dY [rows, N_out] 1x128-
    dequantized, W [N_out, K_in] 128x128-dequantized, multiplied as they are
    (no transpose); returns (C, S) [rows, K_in]."""
    from oracle import gemm
    dY = gemm.dequant_1x128(qdy, sdy)
    W = gemm.dequant_128x128(qw, sw)
    return dY @ W, np.abs(dY) @ np.abs(W)


def _dx_reference(qdy, sdy, qw, sw, block_expert):
    """_dx_rows over the contiguous layout, plus the S_trunc term of the
    GPU's product (dY times the transposed weight)."""
    rows_e = np.repeat(np.asarray(block_expert), 128)
    C = np.zeros((qdy.shape[0], qw.shape[2]))
    S = np.zeros_like(C)
    F = TruncRows(C.shape)
    for e in range(qw.shape[0]):
        r = rows_e == e
        if r.any():
            C[r], S[r] = _dx_rows(qdy[r], sdy[:, r], qw[e], sw[e])
            F[r] = ref_blockscaled(qdy[r], sdy[:, r], np.ascontiguousarray(qw[e].T),
                                   np.ascontiguousarray(sw[e].T))[2]
    return C, S, F


def _transposed_weight(qw, sw):
    """W^T per expert: codes [E, K_in, N_out] and 128x128 scales [E, K_in/128,
    N_out/128]; every 128x128 block of W^T holds the elements of one block
    of W, so its scale is that block's scale."""
    return (qw.transpose(1, 2).contiguous(), sw.transpose(1, 2).contiguous())


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(700, 512, 384, 6, 2), (300, 1024, 256, 9, 3)])
def test_data_gradient_through_the_transposed_weight(dev, shape, out_dtype):
    """dX = dY W of a grouped linear layer: the contiguous grouped GEMM with
    the transposed weight codes and scales, against the oracle's dY W."""
    import moe_cases
    from oracle import scaling
    tokens, hidden, inter, experts, topk = shape
    c = inputs.ContiguousCase(tokens=tokens, hidden=hidden, inter=inter, inter2=128,
                              experts=experts, topk=topk, workload=34)
    ids, _, w1, _ = inputs.contiguous_sources(c)
    lay = moe_cases.contiguous_layout(ids, experts)
    g = np.random.default_rng(320)
    dy = g.standard_normal((lay.m_total, inter)).astype(np.float32)
    dy[lay.row_token < 0] = 0.0
    qdy, sdy = scaling.quantize_1x128(dy)
    qw, sw = scaling.quantize_128x128(w1)
    C, S, F = _dx_reference(qdy, sdy, qw, sw, lay.block_expert)
    print(f"data gradient {shape} out={out_dtype}", flush=True)
    tq, ts = _transposed_weight(torch.from_numpy(qw).cuda(), torch.from_numpy(sw).cuda())
    d = fg8.grouped_gemm_fp8_contiguous(torch.from_numpy(qdy).cuda(), torch.from_numpy(sdy).cuda(),
                                        tq, ts, torch.from_numpy(lay.block_expert).cuda(),
                                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    if out_dtype == torch.float32:
        check_f32(d.cpu().numpy(), C, S, inter, "dX", S_flush=F)
    else:
        check_bf16(d.view(torch.int16).cpu().numpy().view(np.uint16), C, S, inter, "dX",
                   S_flush=F)


def test_data_gradient_full_size_sampled(dev):
    """dX = dG W1 at the MoE size (8192 tokens, top-8 of 32 experts; dG
    [rows, 4096], W1 [32, 4096, 7168]): the GPU quantizes dG and W1 and
    transposes W1's codes and scales; the oracle quantizes sampled rows of
    every expert and two 128-column blocks of dX's columns itself."""
    import moe_cases
    from oracle import scaling
    c = inputs.ContiguousCase()
    ids, _, w1, _ = inputs.contiguous_sources(c)
    lay = moe_cases.contiguous_layout(ids, c.experts)
    g = np.random.default_rng(321)
    dy = g.standard_normal((lay.m_total, c.inter)).astype(np.float32)
    dy[lay.row_token < 0] = 0.0
    tq, ts = fg8.fp8_quantize(torch.from_numpy(w1).cuda(), "128x128")
    tq, ts = _transposed_weight(tq, ts)
    qdy, sdy = fg8.fp8_quantize(torch.from_numpy(dy).cuda(), "1x128")
    d = fg8.grouped_gemm_fp8_contiguous(qdy, sdy, tq, ts,
                                        torch.from_numpy(lay.block_expert).cuda(),
                                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    out = d.view(torch.int16).cpu().numpy().view(np.uint16)
    del tq, ts, qdy, sdy, d
    cbs = g.choice(c.hidden // 128, 2, replace=False)
    cols = np.concatenate([np.arange(cb * 128, cb * 128 + 128) for cb in cbs])
    rows_e = np.repeat(lay.block_expert, 128)
    for e in range(c.experts):
        own = np.nonzero(rows_e == e)[0]
        if own.size == 0:
            continue
        rows = np.unique(np.concatenate([own[:4], own[-1:], g.choice(own, 8)]))
        qdy_o, sdy_o = scaling.quantize_1x128(dy[rows])
        W = np.concatenate([scaling.quantize_128x128(w1[e][:, cb * 128:(cb + 1) * 128])[0]
                            for cb in cbs], axis=1)
        sW = np.concatenate([scaling.quantize_128x128(w1[e][:, cb * 128:(cb + 1) * 128])[1]
                             for cb in cbs], axis=1)
        C, S = _dx_rows(qdy_o, sdy_o, W, sW)
        F = ref_blockscaled(qdy_o, sdy_o, W.T.copy(), sW.T.copy())[2]
        check_bf16(out[np.ix_(rows, cols)], C, S, c.inter, f"dX expert {e}", S_flush=F)
