"""Fused exact-attention forward pass for AMD MI355X (gfx950).

The compute lives in libfa_fwd.so (hand-written HIP kernels behind the C
interface of include/fa_fwd.h); this package is its thin Python binding plus
the seeded input generator used by the tests and the benchmark.
"""
from .binding import (EXPORTED, FA_ERR_ALIAS, FA_ERR_ALIGN, FA_ERR_CAUSAL,  # noqa: F401
                      FA_ERR_HEADS, FA_ERR_HIP, FA_ERR_NULL, FA_ERR_SCALE, FA_ERR_SHAPE,
                      FA_ERR_SCRATCH, FA_ERR_SPLITS, FA_ERR_UNSUPPORTED_D, FA_ERR_WORKSPACE, FA_OK, FaError,
                      bwd, bwd_gqa, fa_bwd, fa_bwd_gqa, fa_bwd_gqa_workspace_size,
                      fa_bwd_workspace_size, fa_fp8_v_bytes, fa_fp8_v_scale_bytes,
                      fa_fwd, fa_fwd_f32, fa_fwd_fp8, fa_fwd_fp8_gqa, fa_fwd_gqa, fa_quantize_qk_fp8,
                      fa_quantize_qk_fp8_rotated,
                      fa_quantize_v_fp8, fwd_fp8, quantize_qk_fp8, quantize_v_fp8, fa_fwd_gqa_num_splits, fa_fwd_splitkv,
                      fa_fwd_splitkv_noalloc, fa_fwd_splitkv_noalloc_max_bytes,
                      fa_fwd_splitkv_num_splits, fa_fwd_splitkv_workspace_size, fa_strerror, fwd,
                      fwd_gqa, fwd_splitkv, load)
