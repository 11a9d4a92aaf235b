"""Fine-grained-scaled FP8 GEMM for MI355X (gfx950).

The entry points mirror the C ABI of libfg8.so (include/fg8.h).  Importing
the package does not load the library; the first call does, and raises if it
has not been built.
"""
from ._lib import (  # noqa: F401
    Fg8Error,
    fp8_quantize,
    gemm_fp8_blockscaled,
    gemm_fp8_blockscaled_noalloc,
    gemm_mxfp8,
    gemm_workspace_bytes,
    grouped_gemm_fp8_contiguous,
    grouped_gemm_fp8_contiguous_swiglu,
    grouped_gemm_fp8_kgrouped,
    grouped_gemm_fp8_masked,
    grouped_gemm_mxfp8_contiguous,
    moe_capacity,
    moe_contiguous_layout_fp8,
    tile_choice,
    version,
)
