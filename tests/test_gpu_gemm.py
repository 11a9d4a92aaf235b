"""Dense block-scaled GEMM against the float64 oracle."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_fp8_amd as fg8
import inputs
from oracle import e4m3, gemm, scaling
from parity import check_bf16, check_f32, ref_blockscaled

pytestmark = pytest.mark.gpu


def _quantized(A, B):
    qa, sa = scaling.quantize_1x128(A)
    qb, sb = scaling.quantize_128x128(B)
    return qa, sa, qb, sb


def _gpu(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in arrays]


def _run(qa, sa, qb, sb, out_dtype, guard=0):
    """Run the GEMM on oracle-quantized operands; optionally surround the
    output with sentinel guard bands that must stay untouched."""
    ta, tsa, tb, tsb = _gpu(qa, sa, qb, sb)
    m, n = qa.shape[0], qb.shape[0]
    if guard:
        buf = torch.full((m * n + 2 * guard,), 7.25, dtype=out_dtype, device="cuda")
        out = buf[guard:guard + m * n].view(m, n)
    else:
        out = None
    d = fg8.gemm_fp8_blockscaled(ta, tsa, tb, tsb, out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    if guard:
        assert torch.all(buf[:guard] == 7.25) and torch.all(buf[guard + m * n:] == 7.25)
    if out_dtype == torch.bfloat16:
        return d.view(torch.int16).cpu().numpy().view(np.uint16)
    return d.cpu().numpy()


def _check(d, C, S, K, out_dtype, where, F=0.0):
    if out_dtype == torch.bfloat16:
        check_bf16(d, C, S, K, where, S_flush=F)
    else:
        check_f32(d, C, S, K, where, S_flush=F)


CASES = [
    ("tiny", None, None, None),                  # 64 x 256 x 512, one x100 outlier row
    ("skinny_a", None, None, None),              # 64 x 2112 x 7168 (split-K)
    ("skinny_b", None, None, None),              # 64 x 24576 x 1536
    ("prefill_a", None, None, None),             # 128 x 7168 x 2048
    ("prefill_b", 300, 1000, 1024),              # several 256 x 128 tiles, ragged M and N
    ("tiny", 1, 1, 128),                         # degenerate
    ("tiny", 17, 130, 256),
    ("prefill_b", 65, 2112, 7168),               # just past the skinny path
    ("skinny_a", 7, 8192, 4096),
    ("tiny", 64, 64, 16384),                     # largest K: 128 K blocks, 8-way split-K
    ("prefill_a", 100, 392, 512),                # 64 < M <= 128 path, ragged M and N
    ("tiny", 64, 256, 32768),                    # long K: 256 K blocks, 8-way split-K
    ("prefill_b", 300, 256, 20480),              # long K on the 128 x 64 tiles
]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name,M,N,K", CASES)
def test_dense_parity(dev, name, M, N, K, out_dtype):
    A, B = inputs.dense_case(name, M, N, K)
    qa, sa, qb, sb = _quantized(A, B)
    C, S, F = ref_blockscaled(qa, sa, qb, sb)
    d = _run(qa, sa, qb, sb, out_dtype, guard=4096)
    _check(d, C, S, A.shape[1], out_dtype, f"{name} {A.shape[0]}x{B.shape[0]}x{A.shape[1]}", F)


def test_dense_prefill_full_size_sampled_rows(dev):
    """4096 x 7168 x 2048 in the launch configuration the benchmark uses;
    the oracle computes 384 sampled rows (every M tile, both ends)."""
    A, B = inputs.dense_case("prefill_b")
    qa, sa, qb, sb = _quantized(A, B)
    d = _run(qa, sa, qb, sb, torch.bfloat16)
    rows = np.unique(np.concatenate([np.arange(0, 4096, 16), [1, 255, 256, 4095],
                                     np.random.default_rng(300).choice(4096, 120)]))
    C, S, F = ref_blockscaled(qa[rows], sa[:, rows], qb, sb)
    check_bf16(d[rows], C, S, 2048, "prefill full size", S_flush=F)


def test_dense_256_tiles_under_one_round_sampled_rows(dev):
    """4096 x 2112 x 7168: 144 tiles of 256 x 256, fewer than the CUs, are
    chosen over 272 tiles of 256 x 128 (which would need a second round);
    the oracle computes 160 sampled rows of the default launch."""
    A, B = inputs.dense_case("prefill_b", 4096, 2112, 7168)
    qa, sa, qb, sb = _quantized(A, B)
    d = _run(qa, sa, qb, sb, torch.bfloat16)
    rows = np.unique(np.concatenate([np.arange(0, 4096, 32), [1, 255, 256, 4095],
                                     np.random.default_rng(302).choice(4096, 28)]))
    C, S, F = ref_blockscaled(qa[rows], sa[:, rows], qb, sb)
    check_bf16(d[rows], C, S, 7168, "4096x2112x7168 sampled", S_flush=F)


def test_quantize_then_gemm_on_gpu(dev):
    """The activation path as the benchmark runs it: the GPU quantizes A and
    B, the GEMM consumes them; the oracle quantizes and multiplies on its own."""
    A, B = inputs.dense_case("skinny_a")
    ta, tb = _gpu(A, B)
    qa, sa = fg8.fp8_quantize(ta, "1x128")
    qb, sb = fg8.fp8_quantize(tb, "128x128")
    d = fg8.gemm_fp8_blockscaled(qa, sa, qb, sb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    C, S, F = ref_blockscaled(*_quantized(A, B))
    check_bf16(d.view(torch.int16).cpu().numpy().view(np.uint16), C, S, 7168, "quantize+gemm",
               S_flush=F)


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (300, 520, 1024), (128, 7168, 2048)])
def test_integer_exact(dev, M, N, K):
    """Codes of small integers with power-of-two scales: every partial sum is
    exact in FP32, so the FP32 output must equal the oracle exactly."""
    g = np.random.default_rng(301)
    ints = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4])
    code = {int(v): int(e4m3.encode(float(v))) for v in ints}
    lut = np.vectorize(code.get)
    ia, ib = g.choice(ints, (M, K)), g.choice(ints, (N, K))
    qa, qb = lut(ia).astype(np.uint8), lut(ib).astype(np.uint8)
    sa = np.full((K // 128, M), 0.25, np.float32)
    sb = np.full((-(-N // 128), K // 128), 2.0, np.float32)
    d = _run(qa, sa, qb, sb, torch.float32)
    C, _ = gemm.gemm_blockscaled(qa, sa, qb, sb)
    assert np.array_equal(d.astype(np.float64), C)


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (300, 400, 1024)])
def test_scale_indexing(dev, M, N, K):
    """Each A group and each B block carries a distinct power of two
    2^((3 i + 5 kb) mod 9 - 4): a scale read from the wrong row, block or K
    block is off by at least 2x and fails the derived FP32 bound."""
    g = np.random.default_rng(302)
    vals = e4m3.DECODE_TABLE[np.isfinite(e4m3.DECODE_TABLE)]
    small = vals[np.abs(vals) <= 8]          # includes the subnormal codes
    qa = e4m3.encode(g.choice(small, (M, K)))
    qb = e4m3.encode(g.choice(small, (N, K)))
    kbs = K // 128
    sa = np.array([[2.0 ** (((3 * m + 5 * kb) % 9) - 4) for m in range(M)] for kb in range(kbs)],
                  np.float32)
    sb = np.array([[2.0 ** (((3 * nb + 5 * kb) % 9) - 4) for kb in range(kbs)]
                   for nb in range(-(-N // 128))], np.float32)
    d = _run(qa, sa, qb, sb, torch.float32)
    C, S, F = ref_blockscaled(qa, sa, qb, sb)
    check_f32(d, C, S, K, "scale indexing", S_flush=F)


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (64, 24576, 1536), (4096, 512, 2048)])
def test_deterministic(dev, M, N, K):
    """Two runs give the same bits (the split-K reduction has a fixed order)."""
    A, B = inputs.dense_case("skinny_a", M, N, K)
    ta, tb = _gpu(A, B)
    qa, sa = fg8.fp8_quantize(ta, "1x128")
    qb, sb = fg8.fp8_quantize(tb, "128x128")
    d1 = fg8.gemm_fp8_blockscaled(qa, sa, qb, sb, out_dtype=torch.float32)
    d2 = fg8.gemm_fp8_blockscaled(qa, sa, qb, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int32), d2.view(torch.int32))


def test_abi_errors_do_not_launch(dev):
    a = torch.zeros((64, 200), dtype=torch.uint8, device="cuda")
    with pytest.raises(fg8.Fg8Error) as e:
        fg8._lib._check(fg8._lib.lib().gemm_fp8_blockscaled(
            fg8._lib._ptr(a), fg8._lib._ptr(a), fg8._lib._ptr(a), fg8._lib._ptr(a),
            fg8._lib._ptr(a), 0, 64, 64, 200, None, 0, None))
    assert e.value.status == fg8._lib.FG8_EUNSUPPORTED and "multiple of 128" in str(e.value)


@pytest.mark.parametrize("name,M,N,K", [
    ("skinny_a", 64, 2112, 7168),    # 48-column wave tiles straddle 128-column B blocks
    ("tiny", 17, 130, 256),          # ragged N, one partial B block
    ("prefill_b", 300, 1000, 1024),  # several tiles in M, split-K
    ("skinny_a", 64, 2112, 1152),    # 9 K blocks
    ("tiny", 17, 130, 640),          # 5 K blocks, ragged M and N
    ("tiny", 33, 200, 128),          # one K block: fewer than the prologue's three stages
    ("skinny_b", 64, 1000, 384),     # three K blocks: exactly the prologue
])
def test_dense_64x96_tiles(dev, monkeypatch, name, M, N, K):
    """The 64 x 96 configuration (index 18 of the compiled list, forced by the
    tuning hook): each wave keeps the scales of both 128-column B blocks its
    columns can touch and applies them per 16-column tile; four stages of one
    K block, so units with fewer K blocks than the prologue's three stages,
    and split-K units, are covered."""
    monkeypatch.setenv("FG8_TILE_OVERRIDE", "18")
    test_dense_parity(dev, name, M, N, K, torch.bfloat16)
