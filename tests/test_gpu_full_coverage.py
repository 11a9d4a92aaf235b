"""Every output element of full-size launches, checked exactly.

Operands are e4m3 codes of integers in [-4, 4] with unit scales.  With
K = 256 every partial sum is an integer of magnitude at most 4096, so the
FP32 output must equal the integer product exactly, as the oracle's
integer-exact GEMM pin states; the reference is a float32 product of the same
integers, which is exact too.  At these sizes the launches use the 256 x 256
tiles in their XCD-blocked order (several whole rounds of the persistent
grid), the contiguous layout's pair and half-height units and the masked
layout's device-side tile enumeration, so a tile that is skipped, computed
for the wrong expert or written twice shows up as a wrong element."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
from moe_grouped_gemm_fp8_amd import inputs
from oracle import e4m3

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
    lay = inputs.contiguous_layout(inputs.zipf_topk_routing(c.workload, c.tokens, c.experts,
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
