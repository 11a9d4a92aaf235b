"""Pins for the oracle's GEMMs (CPU only): exact rational brute force,
identity and one-hot products, an integer-exact product, an element-by-element
restatement of the scale indexing, and the grouped and MX forms reduced to
the dense form."""
from fractions import Fraction

import numpy as np
import torch

from oracle import e4m3, gemm, scaling


def _rand_codes(g, shape):
    codes = g.integers(0, 256, size=shape).astype(np.uint8)
    codes[np.isin(codes, e4m3.NAN_CODES)] = 0x38
    return codes


def _pow2_scales(g, shape, lo=-6, hi=6):
    return (2.0 ** g.integers(lo, hi, size=shape)).astype(np.float32)


def test_fraction_brute_force():
    """4x4x256 with random codes and non-power-of-two scales, summed exactly
    with rationals, against the float64 oracle."""
    g = np.random.default_rng(10)
    M, N, K = 4, 4, 256
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (N, K))
    sa = g.uniform(0.01, 3, (K // 128, M)).astype(np.float32)
    sb = g.uniform(0.01, 3, (1, K // 128)).astype(np.float32)
    C, S = gemm.gemm_blockscaled(qa, sa, qb, sb)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            base = Fraction(0)
            for k in range(K):
                a = Fraction(float(e4m3.DECODE_TABLE[qa[m, k]])) * Fraction(float(sa[k // 128, m]))
                b = Fraction(float(e4m3.DECODE_TABLE[qb[n, k]])) * Fraction(float(sb[n // 128, k // 128]))
                exact += a * b
                base += abs(a * b)
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(1, 10 ** 12) * base
            assert abs(Fraction(S[m, n]) - base) <= Fraction(1, 10 ** 12) * base


def test_scale_indexing_elementwise():
    """Distinct power-of-two scales per A group and per B block; the vectorised
    oracle must equal a plain triple loop that indexes sa[k//128, m] and
    sb[n//128, k//128] directly (a transposed or shifted index fails by >= 2x)."""
    g = np.random.default_rng(11)
    M, N, K = 3, 260, 384
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (N, K))
    sa = np.array([[2.0 ** (((3 * m + 5 * kb) % 9) - 4) for m in range(M)]
                   for kb in range(K // 128)], np.float32)
    sb = np.array([[2.0 ** (((3 * nb + 5 * kb) % 9) - 4) for kb in range(K // 128)]
                   for nb in range(-(-N // 128))], np.float32)
    C, _ = gemm.gemm_blockscaled(qa, sa, qb, sb)
    dec = e4m3.DECODE_TABLE
    for m in range(M):
        for n in (0, 1, 127, 128, 200, 256, 259):
            ref = 0.0
            for k in range(K):
                ref += dec[qa[m, k]] * float(sa[k // 128, m]) * dec[qb[n, k]] * float(sb[n // 128, k // 128])
            assert abs(C[m, n] - ref) <= 1e-12 * max(1.0, abs(ref)), (m, n)


def test_identity_and_one_hot():
    g = np.random.default_rng(12)
    K, N = 256, 300
    qa = np.zeros((K, K), np.uint8)
    np.fill_diagonal(qa, 0x38)                       # 1.0
    sa = np.ones((K // 128, K), np.float32)
    qb = _rand_codes(g, (N, K))
    sb = g.uniform(0.5, 2, (-(-N // 128), K // 128)).astype(np.float32)
    C, S = gemm.gemm_blockscaled(qa, sa, qb, sb)
    B = gemm.dequant_128x128(qb, sb)
    assert np.array_equal(C, B.T)
    # one-hot rows with a scale pick one scaled column of B^T
    qa = np.zeros((5, K), np.uint8)
    picks = [0, 127, 128, 200, 255]
    for r, k in enumerate(picks):
        qa[r, k] = 0x40                              # 2.0
    sa = np.full((K // 128, 5), 0.25, np.float32)
    C, _ = gemm.gemm_blockscaled(qa, sa, qb, sb)
    for r, k in enumerate(picks):
        assert np.array_equal(C[r], 0.5 * B[:, k])


def test_integer_exact_product():
    """Codes of small integers with power-of-two scales: every partial sum is
    an exact dyadic rational, so the oracle equals an int64 matmul exactly."""
    g = np.random.default_rng(13)
    M, N, K = 33, 140, 512
    ints = np.arange(-4, 5)
    code_of = {int(v): int(e4m3.encode(float(v))) for v in ints}
    ia, ib = g.choice(ints, (M, K)), g.choice(ints, (N, K))
    qa = np.vectorize(code_of.get)(ia).astype(np.uint8)
    qb = np.vectorize(code_of.get)(ib).astype(np.uint8)
    sa = np.full((K // 128, M), 0.5, np.float32)
    sb = np.full((-(-N // 128), K // 128), 4.0, np.float32)
    C, S = gemm.gemm_blockscaled(qa, sa, qb, sb)
    assert np.array_equal(C, 2.0 * (ia @ ib.T))
    assert np.array_equal(S, 2.0 * (np.abs(ia) @ np.abs(ib).T))


def test_contiguous_reduces_to_dense_per_block():
    g = np.random.default_rng(14)
    E, N, K = 3, 160, 256
    be = np.array([0, 0, 2, 1, 1, 1], np.int32)
    M = be.size * 128
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (E, N, K))
    sa = g.uniform(0.1, 2, (K // 128, M)).astype(np.float32)
    sb = g.uniform(0.1, 2, (E, 2, K // 128)).astype(np.float32)
    C, S = gemm.grouped_contiguous(qa, sa, qb, sb, be)
    for i, e in enumerate(be):
        r = slice(i * 128, (i + 1) * 128)
        Cd, Sd = gemm.gemm_blockscaled(qa[r], sa[:, r], qb[e], sb[e])
        assert np.array_equal(C[r], Cd) and np.array_equal(S[r], Sd)


def test_masked_defines_only_valid_rows():
    g = np.random.default_rng(15)
    E, cap, N, K = 3, 128, 96, 256
    valid = np.array([0, 128, 37], np.int32)
    qa, qb = _rand_codes(g, (E, cap, K)), _rand_codes(g, (E, N, K))
    sa = g.uniform(0.1, 2, (E, K // 128, cap)).astype(np.float32)
    sb = g.uniform(0.1, 2, (E, 1, K // 128)).astype(np.float32)
    C, _ = gemm.grouped_masked(qa, sa, qb, sb, valid)
    assert np.all(np.isnan(C[0])) and not np.any(np.isnan(C[1]))
    assert not np.any(np.isnan(C[2, :37])) and np.all(np.isnan(C[2, 37:]))
    Cd, _ = gemm.gemm_blockscaled(qa[2], sa[2], qb[2], sb[2])
    assert np.array_equal(C[2, :37], Cd[:37])


def test_mx_equals_blockscaled_with_matching_pow2_scales():
    """An MX product whose E8M0 bytes are constant per 128 columns equals the
    block-scaled product with those powers of two as FP32 scales."""
    g = np.random.default_rng(16)
    G, M, N, K = 2, 40, 130, 256
    qa, qb = _rand_codes(g, (G, M, K)), _rand_codes(g, (G, N, K))
    ja = g.integers(-5, 5, (G, M, K // 128))
    jb = g.integers(-5, 5, (G, 1, K // 128)).repeat(N, axis=1)
    jb[:, 128:] = g.integers(-5, 5, (G, 1, K // 128))
    ea = (np.repeat(ja, 4, axis=-1) + 127).astype(np.uint8)
    eb = (np.repeat(jb, 4, axis=-1) + 127).astype(np.uint8)
    C, S = gemm.gemm_mx(qa, ea, qb, eb)
    for i in range(G):
        sa = np.ascontiguousarray((2.0 ** ja[i]).T).astype(np.float32)
        sb = (2.0 ** jb[i][[0, 128]]).astype(np.float32)
        Cd, Sd = gemm.gemm_blockscaled(qa[i], sa, qb[i], sb)
        assert np.array_equal(C[i], Cd) and np.array_equal(S[i], Sd)
    C2, _ = gemm.gemm_mx(qa, ea, qb, eb, valid=np.array([0, 7]))
    assert np.all(np.isnan(C2[0])) and np.array_equal(C2[1, :7], C[1, :7])
    assert np.all(np.isnan(C2[1, 7:]))


def test_mx_scale_per_32_columns():
    """Each 32-column block carries its own exponent: a one-hot row that
    picks column k sees exactly 2^(ea[k//32] - 127) * 2^(eb[n, k//32] - 127)."""
    K, N = 128, 3
    qa = np.zeros((1, 4, K), np.uint8)
    for r, k in enumerate([0, 31, 32, 127]):
        qa[0, r, k] = 0x38
    ea = np.zeros((1, 4, K // 32), np.uint8) + np.arange(4, dtype=np.uint8) + 120
    qb = np.full((1, N, K), 0x38, np.uint8)
    eb = (np.arange(N * 4).reshape(1, N, 4) + 110).astype(np.uint8)
    C, _ = gemm.gemm_mx(qa, ea, qb, eb)
    for r, k in enumerate([0, 31, 32, 127]):
        for n in range(N):
            want = 2.0 ** (int(ea[0, r, k // 32]) - 127 + int(eb[0, n, k // 32]) - 127)
            assert C[0, r, n] == want


def test_round_to_bf16_against_torch():
    g = np.random.default_rng(17)
    c = np.concatenate([g.standard_normal(100000) * 10.0 ** g.uniform(-6, 6, 100000)])
    c32 = c.astype(np.float32)
    ref = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(gemm.round_to_bf16(c32.astype(np.float64)), ref)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert gemm.round_to_bf16(1 + 2.0 ** -8) == 1.0
    assert gemm.round_to_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert gemm.round_to_bf16(-(1 + 2.0 ** -8)) == -1.0


def test_quantize_then_gemm_tracks_fp32_product():
    """End to end sanity: with fine-grained scales the quantized product stays
    close to the float64 product of the unquantized inputs (e4m3 keeps ~3
    mantissa bits, so the relative error per term is at most 2^-4 per operand)."""
    g = np.random.default_rng(18)
    A = g.standard_normal((16, 512)).astype(np.float32)
    B = (g.standard_normal((64, 512)) / np.sqrt(512)).astype(np.float32)
    qa, sa = scaling.quantize_1x128(A)
    qb, sb = scaling.quantize_128x128(B)
    C, S = gemm.gemm_blockscaled(qa, sa, qb, sb)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.all(np.abs(C - ref) <= 0.13 * S + 1e-12)


def test_contiguous_mx_reduces_to_mx_per_block():
    """Each 128-row block of the MXFP8 contiguous product is the MX product of
    those rows with its expert's B; blocks with an out-of-range id stay
    undefined (NaN)."""
    g = np.random.default_rng(17)
    E, N, K = 3, 96, 256
    be = np.array([2, 0, 0, 5, 1], np.int32)          # id 5 is out of range
    M = be.size * 128
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (E, N, K))
    ea = g.integers(110, 140, (M, K // 32)).astype(np.uint8)
    eb = g.integers(110, 140, (E, N, K // 32)).astype(np.uint8)
    C, S = gemm.grouped_contiguous_mx(qa, ea, qb, eb, be)
    for i, e in enumerate(be):
        r = slice(i * 128, (i + 1) * 128)
        if e >= E:
            assert np.all(np.isnan(C[r])) and np.all(np.isnan(S[r]))
            continue
        Cd, Sd = gemm.gemm_mx(qa[None, r], ea[None, r], qb[None, e], eb[None, e])
        assert np.array_equal(C[r], Cd[0]) and np.array_equal(S[r], Sd[0])


def test_contiguous_mx_equals_blockscaled_with_unit_scales():
    """With every E8M0 byte 127 (scale 1) the MX contiguous product equals the
    block-scaled contiguous product with unit FP32 scales."""
    g = np.random.default_rng(18)
    E, N, K = 2, 130, 256
    be = np.array([1, 0, 1], np.int32)
    M = be.size * 128
    qa, qb = _rand_codes(g, (M, K)), _rand_codes(g, (E, N, K))
    C, S = gemm.grouped_contiguous_mx(qa, np.full((M, K // 32), 127, np.uint8), qb,
                                      np.full((E, N, K // 32), 127, np.uint8), be)
    Cb, Sb = gemm.grouped_contiguous(qa, np.ones((K // 128, M), np.float32), qb,
                                     np.ones((E, 2, K // 128), np.float32), be)
    assert np.array_equal(C, Cb) and np.array_equal(S, Sb)
