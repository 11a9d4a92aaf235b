"""gemm_fp8_blockscaled_noalloc (the entry point that allocates nothing)
through the C ABI, against gemm_fp8_blockscaled on the same operands: two
calls in a row, the second on a smaller problem, must give the same bits as
the entry point with a caller-owned workspace (same kernels, same summation
order), so the scratch array is set up, used, and left reusable."""
import ctypes

import numpy as np
import pytest
import torch

import inputs
from moe_grouped_gemm_fp8_amd import _lib

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def _operands(name, M, N, K):
    A, B = inputs.dense_case(name, M, N, K)
    L = _lib.lib()
    dev = "cuda"
    tA, tB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    qb = torch.empty((N, K), dtype=torch.uint8, device=dev)
    sb = torch.empty((-(-N // 128), K // 128), dtype=torch.float32, device=dev)
    st = P(torch.cuda.current_stream().cuda_stream)
    assert L.fp8_quantize(P(tA.data_ptr()), 1, M, K, 0, P(qa.data_ptr()), P(sa.data_ptr()), st) == 0
    assert L.fp8_quantize(P(tB.data_ptr()), 1, N, K, 1, P(qb.data_ptr()), P(sb.data_ptr()), st) == 0
    return qa, sa, qb, sb


def _both(qa, sa, qb, sb, out):
    """(no-alloc result, workspace result) bits of one product."""
    L = _lib.lib()
    M, K = qa.shape
    N = qb.shape[0]
    st = P(torch.cuda.current_stream().cuda_stream)
    d_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda").to(
        torch.bfloat16 if out == 1 else torch.float32)
    d_ws = d_na.clone()
    args = (P(qa.data_ptr()), P(sa.data_ptr()), P(qb.data_ptr()), P(sb.data_ptr()))
    st_na = L.gemm_fp8_blockscaled_noalloc(*args, P(d_na.data_ptr()), out, M, N, K, st)
    assert st_na == 0, L.fg8_last_error()
    need = L.fg8_gemm_workspace_bytes(M, N, K)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda")
    st_ws = L.gemm_fp8_blockscaled(*args, P(d_ws.data_ptr()), out, M, N, K, P(ws.data_ptr()),
                                   ctypes.c_size_t(ws.numel()), st)
    assert st_ws == 0, L.fg8_last_error()
    torch.cuda.synchronize()
    view = torch.int16 if out == 1 else torch.int32
    return d_na.view(view).cpu().numpy(), d_ws.view(view).cpu().numpy(), need


@pytest.mark.parametrize("out", [0, 1])
def test_noalloc_matches_the_workspace_entry_point(dev, out):
    # 64 x 2112 x 7168 (split-K through the scratch), then a smaller split-K
    # problem that reuses the counters the first call left at zero
    for name, M, N, K in (("skinny_a", 64, 2112, 7168), ("tiny", 40, 520, 2048)):
        qa, sa, qb, sb = _operands(name, M, N, K)
        got, want, need = _both(qa, sa, qb, sb, out)
        print(f"noalloc {M}x{N}x{K} out={out}: split-K scratch {need} bytes", flush=True)
        assert need > 0, "the case must go through the split-K scratch"
        assert np.array_equal(got, want), f"{M}x{N}x{K}: {np.count_nonzero(got != want)} differ"


def test_noalloc_without_split_k(dev):
    """A shape with no split-K (64 x 24576 x 1536: 256 unsplit units) does
    not touch the scratch at all."""
    qa, sa, qb, sb = _operands("skinny_b", 64, 24576, 1536)
    got, want, need = _both(qa, sa, qb, sb, 1)
    assert need == 0 and np.array_equal(got, want)
