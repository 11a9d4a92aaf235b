"""The host tile heuristic through the C ABI (no GPU call): which tile,
split count, launch width and tile order each workload gets on a 256-CU
device.  These are the launch configurations the GPU parity tests and the
benchmark rely on."""
import ctypes

import pytest

from moe_grouped_gemm_fp8_amd import _lib

CUS = 256
DENSE, CONTIGUOUS, MASKED, KGROUPED = 0, 1, 2, 3


def choice(mode, m, n, k, groups=1, cus=CUS):
    out = (ctypes.c_int32 * 5)()
    st = _lib.lib().fg8_tile_choice(mode, m, n, k, groups, cus, ctypes.cast(out, ctypes.c_void_p))
    assert st == 0, _lib.lib().fg8_last_error()
    return tuple(out)   # (tile rows, tile cols, splits, workgroups, tile-order group)


def test_decode_gemm_64x2112x7168():
    # 64 x 32 tiles, two workgroups per CU, split along K: 66 tiles x 7 splits
    bm, bn, splits, grid, raster = choice(DENSE, 64, 2112, 7168)
    assert (bm, bn, raster) == (64, 32, 0)
    assert splits == 7 and grid == 66 * 7


def test_decode_gemm_64x24576x1536_uses_64x96_tiles():
    assert choice(DENSE, 64, 24576, 1536) == (64, 96, 1, 256, 0)


def test_dense_256x256_tiles_when_they_fill_the_chip():
    assert choice(DENSE, 4096, 7168, 2048) == (256, 256, 1, 256, 4)


def test_dense_256x256_tiles_under_one_round():
    # 144 tiles of 256 x 256 against 272 of 256 x 128 (which need a second round)
    assert choice(DENSE, 4096, 2112, 7168) == (256, 256, 1, 144, 4)
    # 192 tiles of 256 x 128 fit in one round: those stay
    assert choice(DENSE, 4096, 1536, 7168)[:2] == (256, 128)


def test_grouped_layouts():
    bm, bn, _, grid, raster = choice(CONTIGUOUS, 67712, 4096, 7168)
    assert (bm, bn, grid, raster) == (256, 256, 256, 4)
    assert choice(MASKED, 256, 4096, 7168, groups=16)[:2] == (256, 256)
    assert choice(MASKED, 80, 160, 384, groups=5)[:2] == (256, 128)   # small: 256 x 128
    assert choice(KGROUPED, 4096, 7168, 67712, groups=32)[:2] == (256, 256)


@pytest.mark.parametrize("args", [(4, 64, 64, 128, 1, CUS), (DENSE, 0, 64, 128, 1, CUS),
                                  (DENSE, 64, 64, 200, 1, CUS), (DENSE, 64, 64, 128, 1, 0),
                                  (MASKED, 64, 64, 128, 0, CUS)])
def test_bad_arguments(args):
    out = (ctypes.c_int32 * 5)()
    assert _lib.lib().fg8_tile_choice(*args, ctypes.cast(out, ctypes.c_void_p)) == 1
    assert _lib.lib().fg8_tile_choice(0, 64, 64, 128, 1, CUS, None) == 1
