"""grouped FP8 block-scaled GEMM for MI355X."""
