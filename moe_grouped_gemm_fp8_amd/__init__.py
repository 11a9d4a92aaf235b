"""Fine-grained-scaled FP8 GEMM for MI355X (gfx950)."""
