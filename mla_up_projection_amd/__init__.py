"""MI355X-native fused MLA query up-projection (GEMM + RoPE/YaRN + MXFP8) and its backward.

The compute lives in libmlaqup.so (hand-written HIP kernels for gfx950, C ABI
in include/mla_qup.h); `binding` marshals torch device tensors into it.
"""
from .binding import (  # noqa: F401
    DTYPE_BF16, DTYPE_FP32, DTYPE_MXFP8, FMT_BSHD, FMT_SBHD, FMT_THD, FUNCTIONS, LIB_PATH, MlaError,
    lib, mla_qup_bwd, mla_qup_bwd_mxfp8, mla_qup_bwd_noalloc, mla_qup_bwd_mxfp8_workspace_size, mla_qup_bwd_workspace_size,
    mla_kv_rope, mla_qup_fwd, mla_status_str, mxfp8_quantize, mxfp8_quantize_t, rope_cache_build)
