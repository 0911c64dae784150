"""MI355X-native fused MLA query up-projection (GEMM + RoPE/YaRN + MXFP8) and its backward."""
