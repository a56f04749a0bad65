"""MoE dispatch/combine for AMD Instinct MI355X (gfx950).

The work is done by hand-written HIP kernels in libmoe_dc.so behind the C ABI of
include/moe_dc.h; this package is the thin Python binding (``binding``) and the in-tree
build (``build``).  PyTorch supplies device memory and streams only.
"""
from .binding import (  # noqa: F401
    EXPORTS, MOE_DC_FLAG_CHECK_IDS, MOE_DC_FLAG_SEPARATE_ROUTE, MOE_DTYPE_DEFAULT,
    MOE_DTYPE_E2M1, MOE_DTYPE_E4M3, MOE_DTYPE_E5M2, MOE_DTYPE_INT8, MOE_ERR_DEVICE,
    MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_OK, MOE_SCALE_E8M0,
    MOE_SCALE_FP32, MOE_SCALE_FP32_RECIPROCAL, MOE_SCALES_NONE, MOE_SCALES_PER_EXPERT,
    MOE_SCALES_SCALAR, MOE_SCALES_SHARED, MOE_TOKEN_BF16, MOE_TOKEN_F16, Launch, MoeDcConfig, MoeDcError,
    alloc_dispatch_outputs, token_torch_dtype,
    code_row_elems, code_type, combine, combine_block_count, combine_int8, combine_quantize,
    combine_scatter, dispatch, load_library, make_config, moe_combine, moe_combine_int8,
    moe_combine_quantize, moe_combine_scatter, moe_dc_combine_scatter_workspace_bytes,
    moe_dc_dispatch_workspace_bytes, moe_dc_last_error, moe_dc_scales_per_row,
    moe_dc_validate, moe_dc_version, moe_dispatch, moe_dispatch_no_workspace, prepare_combine, prepare_combine_int8,
    prepare_combine_quantize, prepare_combine_scatter, prepare_dispatch)
