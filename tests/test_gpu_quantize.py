"""Quantize kernels against the oracle, bit for bit (codes and scales)."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
import inputs
from oracle import e4m3, scaling

pytestmark = pytest.mark.gpu


def _hard_values(g, shape):
    """Mixed magnitudes plus the cases the encoder must get right: zeros of
    both signs, FP32 subnormals, exact e4m3 midpoints after scaling, and groups
    whose amax is a power of two times 448."""
    x = (g.standard_normal(shape) * np.exp(g.uniform(-12, 12, shape[:-1] + (1,)))).astype(np.float32)
    flat = x.reshape(-1, x.shape[-1])
    if flat.shape[0] > 3:
        flat[0, :] = 0.0
        flat[1, :] = -0.0
        flat[2, :64] = np.float32(1e-42)          # FP32 subnormal
        flat[2, 64:] = -np.float32(3e-41)
        vals = e4m3.DECODE_TABLE[np.isfinite(e4m3.DECODE_TABLE)]
        mids = ((vals[:-1] + vals[1:]) / 2)[:flat.shape[1]]
        flat[3, :mids.size] = mids
        flat[3, 0] = 448.0                        # amax 448 -> s = 1: midpoints stay midpoints
    return x


def _run(x, kind):
    t = torch.from_numpy(x).cuda()
    q, s = fg8.fp8_quantize(t, kind)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


# (2, 8200, 512): enough rows for one wave per whole row, in a batch of two
@pytest.mark.parametrize("shape", [(1, 128), (37, 384), (3, 130, 256), (64, 7168), (2, 8200, 512)])
def test_1x128_bit_exact(dev, shape):
    x = _hard_values(np.random.default_rng(200), shape)
    q, s = _run(x, "1x128")
    qo, so = scaling.quantize_1x128(x)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("shape", [(1, 128), (200, 256), (2, 300, 384), (128, 1024)])
def test_128x128_bit_exact(dev, shape):
    x = _hard_values(np.random.default_rng(201), shape)
    q, s = _run(x, "128x128")
    qo, so = scaling.quantize_128x128(x)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("shape", [(1, 32), (5, 96), (3, 17, 256), (64, 7168)])
def test_mx_bit_exact(dev, shape):
    x = _hard_values(np.random.default_rng(202), shape)
    q, e = _run(x, "mx")
    qo, eo = scaling.quantize_mx(x)
    assert np.array_equal(e, eo)
    assert np.array_equal(q, qo)


def test_full_size_activation_rows_sampled(dev):
    """The MoE token matrix (8192 x 7168, N(0,1)): every row is quantized on
    the GPU; sampled rows are checked exactly (groups are per row)."""
    x = inputs._normal(inputs.rng(3, 0), (8192, 7168))
    t = torch.from_numpy(x).cuda()
    for kind, fn in (("1x128", scaling.quantize_1x128), ("mx", scaling.quantize_mx)):
        q, s = fg8.fp8_quantize(t, kind)
        torch.cuda.synchronize()
        rows = np.random.default_rng(203).choice(8192, 96, replace=False)
        qo, so = fn(x[rows])
        assert np.array_equal(q.cpu().numpy()[rows], qo)
        if kind == "1x128":
            assert np.array_equal(s.cpu().numpy()[:, rows], so)
        else:
            assert np.array_equal(s.cpu().numpy()[rows], so)


def test_full_size_weight_blocks_sampled(dev):
    """Expert weights 32 x 4096 x 7168 quantized 128x128 on the GPU; sampled
    row blocks of sampled experts checked exactly."""
    w = inputs._normal(inputs.rng(3, 1), (32, 4096, 7168), 7168 ** -0.5)
    t = torch.from_numpy(w).cuda()
    q, s = fg8.fp8_quantize(t, "128x128")
    torch.cuda.synchronize()
    qc, sc = q.cpu().numpy(), s.cpu().numpy()
    g = np.random.default_rng(204)
    for e in g.choice(32, 4, replace=False):
        for rb in g.choice(32, 2, replace=False):
            blk = w[e, rb * 128:(rb + 1) * 128]
            qo, so = scaling.quantize_128x128(blk)
            assert np.array_equal(qc[e, rb * 128:(rb + 1) * 128], qo)
            assert np.array_equal(sc[e, rb], so[0])


def test_repeatable(dev):
    x = _hard_values(np.random.default_rng(205), (300, 1024))
    a = _run(x, "1x128")
    b = _run(x, "1x128")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _to_bf16(x):
    """float32 -> nearest bfloat16 (ties to even) and the float32 it holds;
    the test's inputs only, so plain bit arithmetic is enough (finite x)."""
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("kind", ["1x128", "128x128", "mx"])
@pytest.mark.parametrize("shape", [(5, 256), (2, 130, 384), (64, 7168)])
def test_bf16_source_bit_exact(dev, kind, shape):
    """A BF16 tensor quantizes exactly like its (exactly widened) FP32 value:
    codes and scales equal the oracle's on the widened tensor."""
    bits, wide = _to_bf16(_hard_values(np.random.default_rng(203), shape))
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    q, s = fg8.fp8_quantize(t, kind)
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    ref = {"1x128": scaling.quantize_1x128, "128x128": scaling.quantize_128x128,
           "mx": scaling.quantize_mx}[kind](wide)
    assert np.array_equal(q, ref[0])
    if kind == "mx":
        assert np.array_equal(s, ref[1])
    else:
        assert np.array_equal(s.view(np.uint32), ref[1].view(np.uint32))
