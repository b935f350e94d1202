"""CPU oracle for C = A·Bᵀ — test infrastructure only (see gemm_oracle.c)."""
