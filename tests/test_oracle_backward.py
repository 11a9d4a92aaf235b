"""Pins of oracle/backward.py (no GPU): the transposed quantizer on columns
with a known amax, the K-grouped GEMM against brute force, the dense
block-scaled GEMM it reduces to, and linearity over the groups."""
import numpy as np

from oracle import backward, e4m3, gemm, scaling


def test_transposed_quantize_of_constant_columns():
    v = np.array([3.0, -0.5, 0.0, 1e-3], np.float32)
    x = np.tile(v, (256, 1))                 # every column constant over 256 rows
    q, s = backward.quantize_1x128_transposed(x)
    assert q.shape == (4, 256) and s.shape == (2, 4)
    for c, val in enumerate(v):
        if val == 0:
            assert np.all(q[c] == 0) and np.all(s[:, c] == 1.0)
        else:
            # amax = |val| -> s = |val|/448 and every element hits +-448
            assert np.all(s[:, c] == np.float32(abs(val) / np.float32(448.0)))
            assert np.all(q[c] == (0x7E if val > 0 else 0xFE))


def test_transposed_groups_run_along_rows():
    g = np.random.default_rng(1)
    x = g.standard_normal((256, 3)).astype(np.float32)
    x[5, 1] = 1000.0                          # dominates group 0 of column 1 only
    q, s = backward.quantize_1x128_transposed(x)
    assert s[0, 1] == np.float32(1000.0 / np.float32(448.0))
    assert s[1, 1] < 1.0 and s[0, 0] < 1.0
    assert q[1, 5] == 0x7E


def _brute(qa, sa, qb, sb, k0, k1):
    M, N = qa.shape[0], qb.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            t = 0.0
            for k in range(k0, k1):
                a = e4m3.DECODE_TABLE[qa[m, k]] * float(sa[k // 128, m])
                b = e4m3.DECODE_TABLE[qb[n, k]] * float(sb[k // 128, n])
                t += a * b
            out[m, n] = t
    return out


def test_grouped_k_brute_force_with_an_empty_group():
    g = np.random.default_rng(2)
    qa, sa = scaling.quantize_1x128(g.standard_normal((3, 512)).astype(np.float32))
    qb, sb = scaling.quantize_1x128(g.standard_normal((4, 512)).astype(np.float32) * 7)
    off = [0, 128, 128, 512]
    C, S = backward.grouped_k(qa, sa, qb, sb, off)
    assert C.shape == (3, 3, 4)
    assert np.allclose(C[0], _brute(qa, sa, qb, sb, 0, 128), rtol=1e-12, atol=1e-12)
    assert np.all(C[1] == 0) and np.all(S[1] == 0)
    assert np.allclose(C[2], _brute(qa, sa, qb, sb, 128, 512), rtol=1e-12, atol=1e-12)


def test_one_group_with_block_constant_b_scales_is_the_blockscaled_gemm():
    g = np.random.default_rng(3)
    K, N = 384, 256
    qa, sa = scaling.quantize_1x128(g.standard_normal((5, K)).astype(np.float32))
    qb, sbb = scaling.quantize_128x128(g.standard_normal((N, K)).astype(np.float32))
    sb_rows = np.repeat(sbb, 128, axis=0)[:N].T.copy()      # [K/128, N], constant per block
    C1, S1 = backward.grouped_k(qa, sa, qb, sb_rows, [0, K])
    C0, S0 = gemm.gemm_blockscaled(qa, sa, qb, sbb)
    assert np.array_equal(C1[0], C0) and np.array_equal(S1[0], S0)


def test_groups_partition_the_full_product():
    g = np.random.default_rng(4)
    K = 1024
    qa, sa = scaling.quantize_1x128(g.standard_normal((6, K)).astype(np.float32))
    qb, sb = scaling.quantize_1x128(g.standard_normal((7, K)).astype(np.float32))
    Cg, _ = backward.grouped_k(qa, sa, qb, sb, [0, 256, 256, 640, 1024])
    Cf, _ = backward.grouped_k(qa, sa, qb, sb, [0, K])
    assert np.allclose(Cg.sum(axis=0), Cf[0], rtol=1e-12, atol=1e-12)
