"""MoE dispatch/combine for AMD Instinct MI355X (gfx950).

The work is done by hand-written HIP kernels in libmoe_dc.so behind the C ABI of
include/moe_dc.h; this package is the thin Python binding (``binding``) and the in-tree
build (``build``).  PyTorch supplies device memory and streams only.
"""
from .binding import (  # noqa: F401
    EXPORTS, MOE_ERR_DEVICE, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
    MOE_OK, MoeDcConfig, MoeDcError, alloc_dispatch_outputs, combine, dispatch, load_library,
    make_config, moe_combine, moe_dc_dispatch_workspace_bytes, moe_dc_last_error,
    moe_dc_scales_per_row, moe_dc_validate, moe_dc_version, moe_dispatch)
