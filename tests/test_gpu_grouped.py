"""MoE grouped GEMMs (contiguous and masked layouts) and the MXFP8 GEMM
against the float64 oracle."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
import inputs
import moe_cases
from oracle import e4m3, gemm, scaling
from parity import TruncRows, check_bf16, check_f32, ref_blockscaled, ref_mx

pytestmark = pytest.mark.gpu

SENTINEL_F32 = np.float32(-12345.5)


def _gpu(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in arrays]


def _bits(d):
    if d.dtype == torch.bfloat16:
        return d.view(torch.int16).cpu().numpy().view(np.uint16)
    return d.cpu().numpy()


def _check(d, C, S, K, where, derived=True, F=0.0):
    if d.dtype == np.uint16:
        return check_bf16(d, C, S, K, where, S_flush=F)
    return check_f32(d, C, S, K, where, derived=derived, S_flush=F)


# ------------------------------------------------------------- contiguous
def _small_contiguous(tokens=300, hidden=512, inter=384, experts=6, topk=2):
    c = inputs.ContiguousCase(tokens=tokens, hidden=hidden, inter=inter, inter2=256,
                              experts=experts, topk=topk, workload=31)
    return c, moe_cases.contiguous_case(c)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(300, 512, 384, 6, 2), (700, 1024, 200, 9, 3)])
def test_contiguous_small(dev, shape, out_dtype):
    c, (lay, a1, w1, a2, w2) = _small_contiguous(*shape)
    qa, sa = scaling.quantize_1x128(a1)
    qb, sb = scaling.quantize_128x128(w1)
    C, S = gemm.grouped_contiguous(qa, sa, qb, sb, lay.block_expert)
    ta, tsa, tb, tsb, tbe = _gpu(qa, sa, qb, sb, lay.block_expert)
    d = fg8.grouped_gemm_fp8_contiguous(ta, tsa, tb, tsb, tbe, out_dtype=out_dtype)
    torch.cuda.synchronize()
    F = TruncRows(C.shape)
    for e in range(c.experts):
        rows = np.repeat(lay.block_expert == e, 128)
        if rows.any():
            F[rows] = ref_blockscaled(qa[rows], sa[:, rows], qb[e], sb[e])[2]
    _check(_bits(d), C, S, c.hidden, "contiguous small", F=F)


def test_contiguous_zero_expert_and_padding(dev):
    """Experts with no rows have no blocks; padding rows of A are zero and come
    out as exact zeros."""
    routing = np.array([[0, 2], [2, 3], [0, 3]] * 50, np.int32)     # expert 1 unused
    lay = moe_cases.contiguous_layout(routing, 5)                       # expert 4 unused too
    assert lay.counts[1] == 0 and lay.counts[4] == 0
    x = inputs._normal(inputs.rng(32, 0), (routing.shape[0], 256))
    a = moe_cases.gather_rows(x, lay.row_token)
    w = inputs._normal(inputs.rng(32, 1), (5, 160, 256), 256 ** -0.5)
    qa, sa = scaling.quantize_1x128(a)
    qb, sb = scaling.quantize_128x128(w)
    ta, tsa, tb, tsb, tbe = _gpu(qa, sa, qb, sb, lay.block_expert)
    d = fg8.grouped_gemm_fp8_contiguous(ta, tsa, tb, tsb, tbe, out_dtype=torch.float32)
    torch.cuda.synchronize()
    C, S = gemm.grouped_contiguous(qa, sa, qb, sb, lay.block_expert)
    out = d.cpu().numpy()
    check_f32(out, C, S, 256, "contiguous zero expert")
    assert np.all(out[lay.row_token < 0] == 0)


def test_contiguous_out_of_range_expert_ids_skip_their_block(dev):
    """A 128-row block whose expert id lies outside [0, E) (here -1 and E) is
    skipped: its output rows keep their previous contents; every other block
    is computed as usual."""
    c, (lay, a1, w1, a2, w2) = _small_contiguous(300, 512, 384, 6, 2)
    qa, sa = scaling.quantize_1x128(a1)
    qb, sb = scaling.quantize_128x128(w1)
    C, S = gemm.grouped_contiguous(qa, sa, qb, sb, lay.block_expert)
    be = lay.block_expert.copy()
    bad = np.zeros(be.size, bool)
    bad[0] = bad[-1] = True
    be[0], be[-1] = -1, c.experts
    ta, tsa, tb, tsb, tbe = _gpu(qa, sa, qb, sb, be)
    out = torch.full((qa.shape[0], qb.shape[1]), float(SENTINEL_F32), dtype=torch.float32,
                     device="cuda")
    fg8.grouped_gemm_fp8_contiguous(ta, tsa, tb, tsb, tbe, out=out)
    torch.cuda.synchronize()
    d = out.cpu().numpy()
    rows_bad = np.repeat(bad, 128)
    assert np.all(d[rows_bad] == SENTINEL_F32)
    good = ~rows_bad
    F = TruncRows(C.shape)
    for e in range(c.experts):
        rows = np.repeat((lay.block_expert == e) & ~bad, 128)
        if rows.any():
            F[rows] = ref_blockscaled(qa[rows], sa[:, rows], qb[e], sb[e])[2]
    check_f32(d[good], C[good], S[good], c.hidden, "contiguous good blocks", S_flush=F[good])


@pytest.mark.parametrize("which", ["w1", "w2"])
def test_contiguous_full_size_sampled(dev, which):
    """The MoE workload at full size (8192 tokens, top-8 of 32 experts, Zipf
    popularity; W1 7168 -> 4096 and W2 2048 -> 7168).  The GPU quantizes and
    multiplies everything; the oracle checks sampled rows of every expert
    against two 128-column blocks, quantized by itself from the FP32 sources."""
    c = inputs.ContiguousCase()
    lay, a1, w1, a2, w2 = moe_cases.contiguous_case(c)
    A, W = (a1, w1) if which == "w1" else (a2, w2)
    del a1, w1, a2, w2
    K = A.shape[1]
    tA, tW = _gpu(A, W)
    qa, sa = fg8.fp8_quantize(tA, "1x128")
    qb, sb = fg8.fp8_quantize(tW, "128x128")
    del tA, tW
    tbe = torch.from_numpy(lay.block_expert).cuda()
    d = fg8.grouped_gemm_fp8_contiguous(qa, sa, qb, sb, tbe, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    out = _bits(d)
    g = np.random.default_rng(400)
    N = W.shape[1]
    nbs = g.choice(N // 128, 2, replace=False)
    cols = np.concatenate([np.arange(nb * 128, nb * 128 + 128) for nb in nbs])
    for e in range(c.experts):
        blocks = np.nonzero(lay.block_expert == e)[0]
        if blocks.size == 0:
            continue
        own = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in blocks])
        rows = np.unique(np.concatenate([own[:8], own[-1:], g.choice(own, 8)]))
        qa_o, sa_o = scaling.quantize_1x128(A[rows])
        Bq = [scaling.quantize_128x128(W[e, nb * 128:(nb + 1) * 128]) for nb in nbs]
        qb_o = np.concatenate([q for q, _ in Bq])
        sb_o = np.concatenate([s for _, s in Bq])      # one row of scales per block
        C, S, F = ref_blockscaled(qa_o, sa_o, qb_o, sb_o)
        check_bf16(out[np.ix_(rows, cols)], C, S, K, f"{which} expert {e}", S_flush=F)


# ------------------------------------------------------------- MXFP8 contiguous
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(300, 512, 384, 6, 2), (700, 1024, 200, 9, 3)])
def test_contiguous_mx_small(dev, shape, out_dtype):
    c, (lay, a1, w1, a2, w2) = _small_contiguous(*shape)
    qa, ea = scaling.quantize_mx(a1)
    qb, eb = scaling.quantize_mx(w1)
    C, S = gemm.grouped_contiguous_mx(qa, ea, qb, eb, lay.block_expert)
    ta, tea, tb, teb, tbe = _gpu(qa, ea, qb, eb, lay.block_expert)
    d = fg8.grouped_gemm_mxfp8_contiguous(ta, tea, tb, teb, tbe, out_dtype=out_dtype)
    torch.cuda.synchronize()
    F = TruncRows(C.shape)
    for e in range(c.experts):
        rows = np.repeat(lay.block_expert == e, 128)
        if rows.any():
            F[rows] = ref_mx(qa[rows], ea[rows], qb[e], eb[e])[2]
    _check(_bits(d), C, S, c.hidden, "mx contiguous small", derived=False, F=F)


def test_contiguous_mx_out_of_range_ids_skip_their_block(dev):
    c, (lay, a1, w1, a2, w2) = _small_contiguous(300, 512, 384, 6, 2)
    qa, ea = scaling.quantize_mx(a1)
    qb, eb = scaling.quantize_mx(w1)
    C, S = gemm.grouped_contiguous_mx(qa, ea, qb, eb, lay.block_expert)
    be = lay.block_expert.copy()
    be[1] = -7
    ta, tea, tb, teb, tbe = _gpu(qa, ea, qb, eb, be)
    out = torch.full((qa.shape[0], qb.shape[1]), float(SENTINEL_F32), dtype=torch.float32,
                     device="cuda")
    fg8.grouped_gemm_mxfp8_contiguous(ta, tea, tb, teb, tbe, out=out)
    torch.cuda.synchronize()
    d = out.cpu().numpy()
    bad = np.repeat(np.arange(be.size) == 1, 128)
    assert np.all(d[bad] == SENTINEL_F32)
    check_f32(d[~bad], C[~bad], S[~bad], c.hidden, "mx contiguous good blocks", derived=False)


def test_contiguous_mx_bf16_sources_full_size_sampled(dev):
    """The MXFP8 training pipeline at the MoE W1 size: BF16 activations and
    weights quantized to MXFP8 on the GPU, then the contiguous grouped GEMM.
    The oracle quantizes the same BF16 values (widened) itself and checks
    sampled rows of every expert against two 128-column blocks."""
    c = inputs.ContiguousCase()
    lay, a1, w1, a2, w2 = moe_cases.contiguous_case(c)
    del a2, w2
    tA = torch.from_numpy(a1).cuda().bfloat16()
    tW = torch.from_numpy(w1).cuda().bfloat16()
    A = tA.float().cpu().numpy()               # the BF16 values, widened exactly
    qa, ea = fg8.fp8_quantize(tA, "mx")
    qb, eb = fg8.fp8_quantize(tW, "mx")
    W = tW.float().cpu().numpy()
    del tA, tW, a1, w1
    tbe = torch.from_numpy(lay.block_expert).cuda()
    d = fg8.grouped_gemm_mxfp8_contiguous(qa, ea, qb, eb, tbe, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    out = _bits(d)
    g = np.random.default_rng(402)
    N, K = W.shape[1], A.shape[1]
    nbs = g.choice(N // 128, 2, replace=False)
    cols = np.concatenate([np.arange(nb * 128, nb * 128 + 128) for nb in nbs])
    for e in range(c.experts):
        blocks = np.nonzero(lay.block_expert == e)[0]
        if blocks.size == 0:
            continue
        own = np.concatenate([np.arange(b * 128, b * 128 + 128) for b in blocks])
        rows = np.unique(np.concatenate([own[:8], own[-1:], g.choice(own, 8)]))
        qa_o, ea_o = scaling.quantize_mx(A[rows])
        qb_o, eb_o = scaling.quantize_mx(W[e][cols])
        C, S, F = ref_mx(qa_o, ea_o, qb_o, eb_o)
        check_bf16(out[np.ix_(rows, cols)], C, S, K, f"mx bf16 expert {e}", S_flush=F)


# ------------------------------------------------------------- masked
def _masked_inputs(E, cap, N, K, workload=41, valid=None):
    mc = inputs.MaskedCase(experts=E, cap=cap, N=N, K=K, workload=workload)
    v, a, b = inputs.masked_case(mc)
    if valid is not None:
        v = np.asarray(valid, np.int32)
    return v, a, b


def _poison(qa, sa_or_e, valid, scale_axis_rows):
    """Rows at or past the count hold NaN codes and NaN (or 0xFF) scales: the
    kernel must never let them reach a stored value."""
    qa = qa.copy()
    s = sa_or_e.copy()
    for e, v in enumerate(valid):
        qa[e, v:] = 0x7F
        if scale_axis_rows == "last":
            s[e, :, v:] = np.nan
        else:
            s[e, v:] = 0xFF
    return qa, s


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_masked_small(dev, out_dtype, K=512, E=7, cap=96, N=200,
                      valid=(0, 96, 1, 37, 64, 95, 50)):
    v, a, b = _masked_inputs(E, cap, N, K, valid=valid)
    qa, sa = scaling.quantize_1x128(a)
    qb, sb = scaling.quantize_128x128(b)
    C, S = gemm.grouped_masked(qa, sa, qb, sb, v)
    qa_p, sa_p = _poison(qa, sa, v, "last")
    ta, tsa, tb, tsb, tv = _gpu(qa_p, sa_p, qb, sb, v)
    out = torch.full((E, cap, N), float(SENTINEL_F32), dtype=out_dtype, device="cuda")
    fg8.grouped_gemm_fp8_masked(ta, tsa, tb, tsb, tv, out=out)
    torch.cuda.synchronize()
    d = _bits(out)
    sentinel = _bits(torch.full((1,), float(SENTINEL_F32), dtype=out_dtype))[0]
    for e in range(E):
        assert np.all(d[e, v[e]:] == sentinel), f"expert {e}: rows past the count were written"
        if v[e]:
            F = ref_blockscaled(qa[e, :v[e]], sa[e][:, :v[e]], qb[e], sb[e])[2]
            _check(d[e, :v[e]], C[e, :v[e]], S[e, :v[e]], K, f"masked expert {e}", F=F)


def test_masked_counts_are_clamped(dev):
    """valid_rows entries below 0 act as 0 and entries above cap act as cap."""
    E, cap, N, K = 3, 64, 96, 256
    v_eff = np.array([0, 64, 10], np.int32)
    _, a, b = _masked_inputs(E, cap, N, K, valid=v_eff)
    qa, sa = scaling.quantize_1x128(a)
    qb, sb = scaling.quantize_128x128(b)
    C, S = gemm.grouped_masked(qa, sa, qb, sb, v_eff)
    ta, tsa, tb, tsb = _gpu(qa, sa, qb, sb)
    tv = torch.tensor([-5, 1000, 10], dtype=torch.int32, device="cuda")
    out = torch.full((E, cap, N), float(SENTINEL_F32), dtype=torch.float32, device="cuda")
    fg8.grouped_gemm_fp8_masked(ta, tsa, tb, tsb, tv, out=out)
    torch.cuda.synchronize()
    d = out.cpu().numpy()
    for e in range(E):
        assert np.all(d[e, v_eff[e]:] == SENTINEL_F32), f"expert {e}"
        if v_eff[e]:
            F = ref_blockscaled(qa[e, :v_eff[e]], sa[e][:, :v_eff[e]], qb[e], sb[e])[2]
            check_f32(d[e, :v_eff[e]], C[e, :v_eff[e]], S[e, :v_eff[e]], K, f"clamped {e}",
                      S_flush=F)


def test_masked_all_counts_zero_writes_nothing(dev):
    """Every expert empty: no tile is enumerated and the output keeps its
    sentinel everywhere (the FP8 and the MXFP8 masked paths)."""
    E, cap, N, K = 4, 128, 256, 512
    v = np.zeros(E, np.int32)
    _, a, b = _masked_inputs(E, cap, N, K, valid=np.full(E, cap, np.int32))
    qa, sa = scaling.quantize_1x128(a)
    qb, sb = scaling.quantize_128x128(b)
    ta, tsa, tb, tsb, tv = _gpu(qa, sa, qb, sb, v)
    out = torch.full((E, cap, N), float(SENTINEL_F32), dtype=torch.float32, device="cuda")
    fg8.grouped_gemm_fp8_masked(ta, tsa, tb, tsb, tv, out=out)
    qx, ex = scaling.quantize_mx(a)
    qy, ey = scaling.quantize_mx(b)
    out_mx = torch.full((E, cap, N), float(SENTINEL_F32), dtype=torch.float32, device="cuda")
    tx, tex, ty, tey = _gpu(qx, ex, qy, ey)
    fg8.gemm_mxfp8(tx, tex, ty, tey, tv, out=out_mx)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == SENTINEL_F32)
    assert np.all(out_mx.cpu().numpy() == SENTINEL_F32)


def test_masked_full_size_sampled(dev):
    """16 experts x 256 rows, N=4096, K=7168, counts ~ U{0..256}: all columns
    computed on the GPU, two 128-column blocks of every expert checked."""
    mc = inputs.MaskedCase()
    v, a, b = inputs.masked_case(mc)
    ta, tb = _gpu(a, b)
    qa, sa = fg8.fp8_quantize(ta, "1x128")
    qb, sb = fg8.fp8_quantize(tb, "128x128")
    del ta, tb
    tv = torch.from_numpy(v).cuda()
    out = torch.full((16, 256, 4096), float(SENTINEL_F32), dtype=torch.bfloat16, device="cuda")
    fg8.grouped_gemm_fp8_masked(qa, sa, qb, sb, tv, out=out)
    torch.cuda.synchronize()
    d = _bits(out)
    sentinel = _bits(torch.full((1,), float(SENTINEL_F32), dtype=torch.bfloat16))[0]
    g = np.random.default_rng(401)
    for e in range(16):
        assert np.all(d[e, v[e]:] == sentinel)
        if not v[e]:
            continue
        nbs = g.choice(32, 2, replace=False)
        cols = np.concatenate([np.arange(nb * 128, nb * 128 + 128) for nb in nbs])
        qa_o, sa_o = scaling.quantize_1x128(a[e, :v[e]])
        Bq = [scaling.quantize_128x128(b[e, nb * 128:(nb + 1) * 128]) for nb in nbs]
        C, S, F = ref_blockscaled(qa_o, sa_o, np.concatenate([q for q, _ in Bq]),
                                  np.concatenate([s for _, s in Bq]))
        check_bf16(d[e, :v[e]][:, cols], C, S, 7168, f"masked full expert {e}", S_flush=F)


# ------------------------------------------------------------- MXFP8
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mx_masked_small(dev, out_dtype, K=384, E=5, cap=80, N=160, valid=(80, 0, 33, 1, 79)):
    v, a, b = _masked_inputs(E, cap, N, K, workload=42, valid=valid)
    qa, ea = scaling.quantize_mx(a)
    qb, eb = scaling.quantize_mx(b)
    C, S = gemm.gemm_mx(qa, ea, qb, eb, v)
    qa_p, ea_p = _poison(qa, ea, v, "rows")
    ta, tea, tb, teb, tv = _gpu(qa_p, ea_p, qb, eb, v)
    out = torch.full((E, cap, N), float(SENTINEL_F32), dtype=out_dtype, device="cuda")
    fg8.gemm_mxfp8(ta, tea, tb, teb, tv, out=out)
    torch.cuda.synchronize()
    d = _bits(out)
    sentinel = _bits(torch.full((1,), float(SENTINEL_F32), dtype=out_dtype))[0]
    for e in range(E):
        assert np.all(d[e, v[e]:] == sentinel)
        if v[e]:
            F = ref_mx(qa[e, :v[e]], ea[e, :v[e]], qb[e], eb[e])[2]
            _check(d[e, :v[e]], C[e, :v[e]], S[e, :v[e]], K, f"mx expert {e}", derived=False, F=F)


# capacities above one 256-row tile: each expert spans several tile rows that
# read the same B rows, so the launch copies B without the non-temporal hint
# that one-tile-row capacities get; the counts end in the first, a middle and
# the last tile row
CAP_ABOVE_TILE = dict(E=3, cap=600, N=200, valid=(600, 257, 130))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_masked_capacity_above_one_tile(dev, out_dtype):
    test_masked_small(dev, out_dtype, K=512, **CAP_ABOVE_TILE)
    test_mx_masked_small(dev, out_dtype, K=384, **CAP_ABOVE_TILE)


def test_mx_long_k(dev):
    """MXFP8 with K = 32768 (1024 E8M0 blocks per row), two groups, no mask."""
    g = np.random.default_rng(408)
    G, m, n, K = 2, 40, 96, 32768
    a = g.standard_normal((G, m, K)).astype(np.float32)
    b = (g.standard_normal((G, n, K)) * K ** -0.5).astype(np.float32)
    qa, ea = scaling.quantize_mx(a)
    qb, eb = scaling.quantize_mx(b)
    ta, tea, tb, teb = _gpu(qa, ea, qb, eb)
    d = fg8.gemm_mxfp8(ta, tea, tb, teb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    C, S = gemm.gemm_mx(qa, ea, qb, eb)
    got = d.cpu().numpy()
    for i in range(G):
        check_f32(got[i], C[i], S[i], K, f"mx long K group {i}", derived=False)


def test_mx_dense_and_exponent_spread(dev):
    """valid_rows = NULL means every row; exponents spread over a wide range
    (per-row magnitudes 2^-20 .. 2^20) exercise the E8M0 lane mapping."""
    g = np.random.default_rng(402)
    G, M, N, K = 2, 70, 150, 512
    a = (g.standard_normal((G, M, K)) * 2.0 ** g.integers(-20, 20, (G, M, K // 32)).repeat(32, -1)).astype(np.float32)
    b = (g.standard_normal((G, N, K)) * 2.0 ** g.integers(-20, 20, (G, N, K // 32)).repeat(32, -1)).astype(np.float32)
    qa, ea = scaling.quantize_mx(a)
    qb, eb = scaling.quantize_mx(b)
    C, S = gemm.gemm_mx(qa, ea, qb, eb)
    ta, tea, tb, teb = _gpu(qa, ea, qb, eb)
    d = fg8.gemm_mxfp8(ta, tea, tb, teb, None, out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = check_f32(d.cpu().numpy(), C, S, K, "mx dense", derived=False)
    print(f"\nmx dense, exponent spread +-20: max |err|/S = {err:.2e}")


def test_mx_masked_full_size_sampled(dev):
    """The MXFP8 variant of the masked workload: same FP32 sources, 1x32 E8M0
    scales for A and B, quantized on the GPU; sampled columns checked."""
    mc = inputs.MaskedCase()
    v, a, b = inputs.masked_case(mc)
    ta, tb = _gpu(a, b)
    qa, ea = fg8.fp8_quantize(ta, "mx")
    qb, eb = fg8.fp8_quantize(tb, "mx")
    del ta, tb
    tv = torch.from_numpy(v).cuda()
    out = torch.full((16, 256, 4096), float(SENTINEL_F32), dtype=torch.bfloat16, device="cuda")
    fg8.gemm_mxfp8(qa, ea, qb, eb, tv, out=out)
    torch.cuda.synchronize()
    d = _bits(out)
    sentinel = _bits(torch.full((1,), float(SENTINEL_F32), dtype=torch.bfloat16))[0]
    g = np.random.default_rng(403)
    for e in range(16):
        assert np.all(d[e, v[e]:] == sentinel)
        if not v[e]:
            continue
        cols = g.choice(4096, 96, replace=False)
        qa_o, ea_o = scaling.quantize_mx(a[e:e + 1, :v[e]])
        qb_o, eb_o = scaling.quantize_mx(b[e:e + 1, cols])
        C, S, F = ref_mx(qa_o[0], ea_o[0], qb_o[0], eb_o[0])
        check_bf16(d[e, :v[e]][:, cols], C, S, 7168, f"mx full expert {e}", S_flush=F)


def test_grouped_deterministic(dev):
    v, a, b = _masked_inputs(6, 128, 384, 1024, workload=43)
    qa, sa = scaling.quantize_1x128(a)
    qb, sb = scaling.quantize_128x128(b)
    ta, tsa, tb, tsb, tv = _gpu(qa, sa, qb, sb, v)
    d1 = fg8.grouped_gemm_fp8_masked(ta, tsa, tb, tsb, tv, out_dtype=torch.float32)
    d2 = fg8.grouped_gemm_fp8_masked(ta, tsa, tb, tsb, tv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int32), d2.view(torch.int32))
