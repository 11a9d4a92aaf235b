"""Every output element of full-size launches, checked exactly.

Operands are e4m3 codes of integers in [-4, 4] with unit scales.  With
K = 256 every partial sum is an integer of magnitude at most 4096, so the
FP32 output must equal the integer product exactly, as the oracle's
integer-exact GEMM pin states; the reference is a float32 product of the same
integers, which is exact too.  At these sizes the launches use the 256 x 256
tiles in their XCD-blocked order (several whole rounds of the persistent
grid), the contiguous layout's pair and half-height units and the masked
layout's device-side tile enumeration, so a tile that is skipped, computed
for the wrong expert or written twice shows up as a wrong element.

The MXFP8 launches take E8M0 bytes in {126, 127, 128} (scales 1/2, 1, 2)
drawn per row and 32-element block, and K = 1152: nine K blocks, so the
256 x 256 MXFP8 tiles fetch their scales in three groups of four K blocks
(the first group buffer is reused and the last group is partial).  Every
product is then a multiple of 1/4 below 64, each 16-wide group sum lies
within 2^12 of its quantum and every partial sum is a multiple of 1/4 below
2^17, so the FP32 output is exact again and a scale taken from the wrong
row, block or group buffer shows up as a wrong element.  The reference is
the float64 product of the dequantized operands, which is exact."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
import inputs
import moe_cases
from oracle import e4m3
from parity import Trunc, check_swiglu_quant

pytestmark = pytest.mark.gpu

K = 256
NAN_CODE = 0x7F


def _ints(g, shape):
    return g.integers(-4, 5, size=shape).astype(np.float32)


def _codes(x):
    return torch.from_numpy(e4m3.encode(x)).cuda()


def _ones(*shape):
    return torch.ones(shape, dtype=torch.float32, device="cuda")


def _exact(got, want, where):
    bad = np.count_nonzero(got != want)
    assert bad == 0, f"{where}: {bad} of {want.size} elements differ"


def test_dense_8192x7168(dev):
    M, N = 8192, 7168
    g = np.random.default_rng(701)
    a, b = _ints(g, (M, K)), _ints(g, (N, K))
    print(f"full coverage dense {M}x{N}x{K}", flush=True)
    d = fg8.gemm_fp8_blockscaled(_codes(a), _ones(K // 128, M), _codes(b),
                                 _ones((N + 127) // 128, K // 128), out_dtype=torch.float32)
    torch.cuda.synchronize()
    _exact(d.cpu().numpy(), a @ b.T, "dense")


def test_contiguous_full_layout(dev):
    """The 8192-token top-8 of 32 Zipf routing layout (about 67.7k rows, expert
    boundaries at arbitrary 128-row blocks), N = 1024."""
    c = inputs.ContiguousCase()
    lay = moe_cases.contiguous_layout(inputs.zipf_topk_routing(c.workload, c.tokens, c.experts,
                                                            c.topk), c.experts)
    M, N, E = lay.m_total, 1024, c.experts
    be = lay.block_expert
    g = np.random.default_rng(702)
    a, b = _ints(g, (M, K)), _ints(g, (E, N, K))
    print(f"full coverage contiguous {M}x{N}x{K}, {E} experts", flush=True)
    d = fg8.grouped_gemm_fp8_contiguous(_codes(a), _ones(K // 128, M), _codes(b),
                                        _ones(E, (N + 127) // 128, K // 128),
                                        torch.from_numpy(be).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    want = np.empty((M, N), np.float32)
    rows_e = np.repeat(be, 128)
    for e in range(E):
        r = rows_e == e
        if r.any():
            want[r] = a[r] @ b[e].T
    _exact(got, want, "contiguous")


def test_masked_wide(dev):
    """16 experts x 256 rows, counts ~ U{0..256}, N = 8192: rows past each
    count hold NaN codes and must keep the sentinel."""
    mc = inputs.MaskedCase()
    E, cap, N = mc.experts, mc.cap, 8192
    v = inputs.masked_case_counts(mc)
    g = np.random.default_rng(703)
    a, b = _ints(g, (E, cap, K)), _ints(g, (E, N, K))
    qa = e4m3.encode(a)
    for e in range(E):
        qa[e, v[e]:] = NAN_CODE
    sentinel = -12345.0
    out = torch.full((E, cap, N), sentinel, dtype=torch.float32, device="cuda")
    print(f"full coverage masked {E}x{cap}x{N}x{K}, valid {int(v.sum())}", flush=True)
    fg8.grouped_gemm_fp8_masked(torch.from_numpy(qa).cuda(), _ones(E, K // 128, cap), _codes(b),
                                _ones(E, (N + 127) // 128, K // 128),
                                torch.from_numpy(v.astype(np.int32)).cuda(),
                                out_dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for e in range(E):
        _exact(got[e, :v[e]], a[e, :v[e]] @ b[e].T, f"masked expert {e}")
        assert (got[e, v[e]:] == sentinel).all(), f"masked expert {e}: rows past the count written"


MX_K = 1152


def _e8m0(g, shape):
    return g.integers(126, 129, size=shape).astype(np.uint8)


def _mx_value(ints, e):
    """ints [..., K] times 2^(e - 127) per 32-element block, float64 (exact)."""
    return ints.astype(np.float64) * np.repeat(np.exp2(e.astype(np.float64) - 127.0), 32, axis=-1)


def test_mx_masked_wide(dev):
    """MXFP8 masked layout at full width: 16 experts x 256 rows, counts ~
    U{0..256}, N = 8192; rows past each count hold NaN codes and NaN (0xFF)
    scale bytes and must keep the sentinel."""
    mc = inputs.MaskedCase()
    E, cap, N = mc.experts, mc.cap, 8192
    v = inputs.masked_case_counts(mc)
    g = np.random.default_rng(704)
    a, b = _ints(g, (E, cap, MX_K)), _ints(g, (E, N, MX_K))
    ea, eb = _e8m0(g, (E, cap, MX_K // 32)), _e8m0(g, (E, N, MX_K // 32))
    qa = e4m3.encode(a)
    ea_dev = ea.copy()
    for e in range(E):
        qa[e, v[e]:] = NAN_CODE
        ea_dev[e, v[e]:] = 0xFF
    sentinel = -12345.0
    out = torch.full((E, cap, N), sentinel, dtype=torch.float32, device="cuda")
    print(f"full coverage mx masked {E}x{cap}x{N}x{MX_K}, valid {int(v.sum())}", flush=True)
    fg8.gemm_mxfp8(torch.from_numpy(qa).cuda(), torch.from_numpy(ea_dev).cuda(), _codes(b),
                   torch.from_numpy(eb).cuda(), torch.from_numpy(v.astype(np.int32)).cuda(),
                   out_dtype=torch.float32, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for e in range(E):
        want = _mx_value(a[e, :v[e]], ea[e, :v[e]]) @ _mx_value(b[e], eb[e]).T
        _exact(got[e, :v[e]].astype(np.float64), want, f"mx masked expert {e}")
        assert (got[e, v[e]:] == sentinel).all(), f"mx masked expert {e}: rows past the count"


def test_mx_contiguous_full_layout(dev):
    """MXFP8 contiguous layout over the full 8192-token top-8 of 32 routing
    layout (about 67.7k rows), N = 1024."""
    c = inputs.ContiguousCase()
    lay = moe_cases.contiguous_layout(inputs.zipf_topk_routing(c.workload, c.tokens, c.experts,
                                                               c.topk), c.experts)
    M, N, E = lay.m_total, 1024, c.experts
    be = lay.block_expert
    g = np.random.default_rng(705)
    a, b = _ints(g, (M, MX_K)), _ints(g, (E, N, MX_K))
    ea, eb = _e8m0(g, (M, MX_K // 32)), _e8m0(g, (E, N, MX_K // 32))
    print(f"full coverage mx contiguous {M}x{N}x{MX_K}, {E} experts", flush=True)
    d = fg8.grouped_gemm_mxfp8_contiguous(_codes(a), torch.from_numpy(ea).cuda(), _codes(b),
                                          torch.from_numpy(eb).cuda(), torch.from_numpy(be).cuda(),
                                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    rows_e = np.repeat(be, 128)
    for e in range(E):
        r = rows_e == e
        if r.any():
            want = _mx_value(a[r], ea[r]) @ _mx_value(b[e], eb[e]).T
            _exact(got[r].astype(np.float64), want, f"mx contiguous expert {e}")


def test_kgrouped_full_layout(dev):
    """The K-grouped weight-gradient GEMM over the expert row ranges of the
    full 8192-token top-8 of 32 routing layout (a few hundred to about 7.9k
    rows per expert), with m = 1024 and n = 512 so that the 256 x 256 tiles
    fill the chip: dW_e = dY_e^T X_e for every expert, every element."""
    c = inputs.ContiguousCase()
    lay = moe_cases.contiguous_layout(inputs.zipf_topk_routing(c.workload, c.tokens, c.experts,
                                                               c.topk), c.experts)
    T, m, n, E = lay.m_total, 1024, 512, c.experts
    off = lay.offsets.astype(np.int32)
    g = np.random.default_rng(706)
    a, b = _ints(g, (m, T)), _ints(g, (n, T))       # dY^T and X^T, tokens along K
    print(f"full coverage k-grouped {E}x{m}x{n} over {T} rows", flush=True)
    d = fg8.grouped_gemm_fp8_kgrouped(_codes(a), _ones(T // 128, m), _codes(b), _ones(T // 128, n),
                                      torch.from_numpy(off).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    for e in range(E):
        k0, k1 = int(off[e]), int(off[e + 1])
        want = a[:, k0:k1].astype(np.float64) @ b[:, k0:k1].astype(np.float64).T
        _exact(got[e].astype(np.float64), want, f"k-grouped expert {e}")


@pytest.mark.timeout(600)
def test_gated_full_layout(dev):
    """The W1 GEMM with the SiLU-gated activation and its 1x128 requantize
    fused, over the full 8192-token top-8 of 32 routing layout, N = 4096
    (2048 columns of h): with integer operands and unit scales every gate and
    up value is an exact integer, so the only error left is the activation's
    FP32 arithmetic (relative 2^-20 in the bounds), and every code and scale
    of h on every row of every expert's blocks is checked against those
    bounds."""
    c = inputs.ContiguousCase()
    lay = moe_cases.contiguous_layout(inputs.zipf_topk_routing(c.workload, c.tokens, c.experts,
                                                               c.topk), c.experts)
    M, N, E = lay.m_total, 4096, c.experts
    be = lay.block_expert
    g = np.random.default_rng(707)
    a, b = _ints(g, (M, K)), _ints(g, (E, N, K))
    print(f"full coverage gated {M}x{N}x{K}, {E} experts", flush=True)
    q, s = fg8.grouped_gemm_fp8_contiguous_swiglu(_codes(a), _ones(K // 128, M), _codes(b),
                                                  _ones(E, N // 128, K // 128),
                                                  torch.from_numpy(be).cuda())
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    rows_e = np.repeat(be, 128)
    moved = 0
    for e in range(E):
        r = np.nonzero(rows_e == e)[0]
        if r.size == 0:
            continue
        C = (a[r] @ b[e].T).astype(np.float64)      # exact: integers below 2^12
        moved += check_swiglu_quant(q[r], s[:, r], C, np.zeros_like(C), Trunc.zeros(C.shape), K,
                                    f"gated expert {e}")
        if e % 8 == 7:
            print(f"  experts 0..{e} checked", flush=True)
    print(f"gated, every element: {moved} codes off the oracle's own rounding of h", flush=True)
