"""The 256 x 256 tile configuration on small, ragged problems.

The library picks 256 x 256 tiles only when they alone cover every CU, so the
full-size tests reach them but the small cases do not.  Here the tuning hook
FG8_TILE_OVERRIDE forces that configuration (index 17 of the compiled list)
on the small dense, contiguous, masked, gated and K-grouped cases, whose
oracle checks are reused unchanged: ragged M and N, odd numbers of 128-row
blocks per expert (a 256-row pair that straddles two experts runs as two
half-height units), skipped blocks, clamped counts and empty groups."""
import pytest
import torch

import test_gpu_backward as B
import test_gpu_gemm as D
import test_gpu_grouped as G
import test_gpu_swiglu as S

pytestmark = pytest.mark.gpu

TILE_256 = "17"


@pytest.fixture
def tiles256(monkeypatch):
    monkeypatch.setenv("FG8_TILE_OVERRIDE", TILE_256)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name,M,N,K", [
    ("prefill_b", 300, 1000, 1024),
    ("tiny", 17, 130, 256),
    ("tiny", 1, 1, 128),
    ("prefill_b", 300, 256, 20480),
])
def test_dense(dev, tiles256, name, M, N, K, out_dtype):
    D.test_dense_parity(dev, name, M, N, K, out_dtype)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(300, 512, 384, 6, 2), (700, 1024, 200, 9, 3)])
def test_contiguous(dev, tiles256, shape, out_dtype):
    G.test_contiguous_small(dev, shape, out_dtype)
    G.test_contiguous_mx_small(dev, shape, out_dtype)


def test_contiguous_mx_partial_scale_group(dev, tiles256):
    """K = 640: five K blocks, so the E8M0 scales end on a partial group of
    the four fetched at a time."""
    G.test_contiguous_mx_small(dev, (300, 640, 384, 6, 2), torch.float32)


def test_contiguous_skipped_blocks(dev, tiles256):
    G.test_contiguous_zero_expert_and_padding(dev)
    G.test_contiguous_out_of_range_expert_ids_skip_their_block(dev)
    G.test_contiguous_mx_out_of_range_ids_skip_their_block(dev)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_masked(dev, tiles256, out_dtype):
    G.test_masked_small(dev, out_dtype)
    G.test_mx_masked_small(dev, out_dtype)
    G.test_masked_capacity_above_one_tile(dev, out_dtype)


@pytest.mark.parametrize("K", [640, 1152, 2048])
def test_mx_masked_scale_groups(dev, tiles256, K):
    """The 256 x 256 MXFP8 tiles fetch E8M0 scales for four K blocks at a
    time: 5 and 9 K blocks end on a partial group, 16 on whole ones."""
    G.test_mx_masked_small(dev, torch.float32, K=K)


@pytest.mark.parametrize("K", [128, 256, 384, 640])
def test_masked_few_k_blocks(dev, tiles256, K):
    """The masked FP32-scaled tiles issue the A part of a stage two K blocks
    ahead: one, two, three and five K blocks cover the pipeline's start and
    end (nothing ahead, one block ahead, an odd tail)."""
    G.test_masked_small(dev, torch.bfloat16, K=K)


@pytest.mark.parametrize("knob", [("FG8_STAGGER", "0"), ("FG8_ROTATE", "1")])
def test_tuning_knobs(dev, tiles256, monkeypatch, knob):
    """The issue-order and K-walk knobs select other code paths in the same
    kernels (every wave issuing a stage at once; each unit starting its K
    walk at a unit-dependent block): same oracle checks."""
    monkeypatch.setenv(*knob)
    D.test_dense_parity(dev, "prefill_b", 300, 1000, 1024, torch.bfloat16)
    G.test_contiguous_small(dev, (700, 1024, 200, 9, 3), torch.bfloat16)
    G.test_masked_small(dev, torch.float32)
    G.test_mx_masked_small(dev, torch.float32, K=1152)
    S.test_swiglu_small(dev, (300, 512, 512, 6, 2))


def test_masked_clamped_counts(dev, tiles256):
    G.test_masked_counts_are_clamped(dev)


@pytest.mark.parametrize("shape", [(300, 512, 512, 6, 2), (700, 1024, 768, 9, 3)])
def test_gated_epilogue(dev, tiles256, shape):
    S.test_swiglu_small(dev, shape)


def test_gated_epilogue_skipped_blocks(dev, tiles256):
    S.test_swiglu_skips_out_of_range_blocks(dev)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", [
    (300, 200, [0, 256, 256, 1024, 1152]),
    (256, 384, [0, 128]),
    (64, 130, [0, 512, 1536, 1536, 1536, 2048]),
])
def test_kgrouped(dev, tiles256, case, out_dtype):
    B.test_kgrouped_small(dev, case, out_dtype)
