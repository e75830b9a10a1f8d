"""CPU oracle of the W4Ax mixed-precision GEMM. TEST INFRASTRUCTURE ONLY."""
