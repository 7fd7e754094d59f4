"""SmoothQuant W8A8 linear layer on MI355X (gfx950): Python binding of libsq.so.

The kernels and the C ABI live in csrc/ and include/sq.h; this package only
marshals torch tensors into those calls (prepared.py saves and loads the
offline products).  Importing it loads the HIP library
and fails if it has not been built.
"""
from .sq import (SQ_BF16, SQ_F32, SQ_I32, SQ_MAX_K, EXPORTED, LIB_PATH,  # noqa: F401
                 SQ_NORM_LAYER, SQ_NORM_RMS, sq_fold_norm_gain, sq_norm_quant_act,
                 sq_decomp_gemm, sq_decomp_prepare_weights, sq_decomp_quant_act, sq_decomp_select,
                 sq_fp8_gemm, sq_quant_act_fp8, sq_quantize_weights_fp8,
                 sq_act_absmax, sq_col_absmax, sq_quant_act, sq_quant_act_per_tensor,
                 sq_quant_act_static, sq_quantize_weights, sq_smooth_scales,
                 sq_smooth_scales_from_absmax, sq_status_string, sq_w8a8_gemm, sq_w8a8_linear,
                 sq_w8a8_linear_workspace_size, sq_w8a8_linear_noalloc,
                 SQ_NOALLOC_SCRATCH_BYTES)
from .prepared import load_prepared, save_prepared  # noqa: F401
