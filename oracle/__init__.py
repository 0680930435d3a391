"""CPU oracle for the FP8 scaled-GEMM path (test infrastructure only)."""
